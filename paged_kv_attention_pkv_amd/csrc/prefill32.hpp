// prefill32.hpp -- device code of the 32-row prefill kernel (head_dim 64 and
// 128; included by prefill.hip and mixed.hip).  What it computes is described
// at the top of prefill.hip.
#pragma once

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {

namespace {

constexpr float kLn2f = 0.6931471805599453f;
constexpr float kNegInff = -__builtin_inff();

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;                   // waves per workgroup
constexpr int kRowsPerWave = 32;            // query rows per wave
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBN = 64;                     // keys per tile (four pages)
constexpr int kThreads = kWaves * kWave;
// A row's running max is raised only when a tile's scores exceed it by more
// than this (log2 units); weights relative to a stale max stay below 2^8, so
// the output (normalised by the same max) is unchanged and the rescale of the
// accumulators is skipped for most tiles.
constexpr float kRescaleSlack = 8.f;

// Key rows are padded by 48 B: row starts then fall 12 banks (of 64) apart,
// which measured fastest for both the K-operand reads and the transposing
// V reads (a 16 B pad left the transposing reads 2-way conflicted).
template <int D, int KPAD = 24, int VPAD = KPAD>
struct Smem {
    static constexpr int KSTRIDE = D + KPAD;          // bf16 elements per K row
    static constexpr int VSTRIDE = D + VPAD;          // and per V row
    static constexpr int VOFF = kBN * KSTRIDE;        // the V tile follows the K tile
    static constexpr int BUF = VOFF + kBN * VSTRIDE;  // K then V, one stage
    static constexpr int BYTES = 2 * BUF * 2;         // two stages of bf16
    static constexpr int STRIDE = KSTRIDE;            // equal pads: one stride for both
    static constexpr int TILE = VOFF;
};

// Global loads of one key tile by a workgroup of NT threads: thread t holds
// chunks t + NT*i (8 dims each) of K and of V; keys past kv are zero.
template <int D, int NT = kThreads>
struct TileRegs {
    static constexpr int CHUNKS = kBN * D / 8 / NT;  // per thread
    u32x4 k[CHUNKS], v[CHUNKS];
};

// The 64 lanes of one wave-instruction load chunks of consecutive keys that
// lie in one page, so each instruction goes through that page's buffer
// resource; its byte range stops at the page's last valid key, so keys at or
// past kv (and whole pages past it) load as zeros, without branches.
template <int D, int NT = kThreads>
__device__ __forceinline__ void load_tile(const PrefillArgs &a, const int32_t *bt, int g, int tile, int kv,
                                          TileRegs<D, NT> &t) {
    constexpr int CPK = D / 8;  // 16-byte chunks per key row
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t tok_bytes = a.s_tok * 2;
    Rsrc rk[kBN / kPage], rv[kBN / kPage];
#pragma unroll
    for (int u = 0; u < kBN / kPage; ++u) {
        const int blk = tile * (kBN / kPage) + u;
        const int valid = min(max(kv - blk * kPage, 0), kPage);
        // 16-token block blk: table column blk >> page_shift, sub-page blk & (2^page_shift - 1)
        int pg = valid > 0 ? bt[blk >> a.page_shift] : 0;
        pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
        const int64_t sub = blk & ((1 << a.page_shift) - 1);
        const int64_t off = ((int64_t)pg * a.s_page + (int64_t)g * a.s_head + sub * kPage * a.s_tok) * 2;
        const int32_t bytes = (int32_t)(valid * tok_bytes);
        rk[u] = make_rsrc((const char *)a.k_cache + off, bytes);
        rv[u] = make_rsrc((const char *)a.v_cache + off, bytes);
    }
#pragma unroll
    for (int i = 0; i < TileRegs<D, NT>::CHUNKS; ++i) {
        const int c0 = kWave * wave + NT * i;  // first chunk of this wave-instruction
        const int u = uniform((c0 / CPK) >> 4);      // its page within the tile
        const int c = c0 + lane;
        const int key = c / CPK;
        const uint32_t voff = (uint32_t)((key & 15) * tok_bytes) + (uint32_t)(c - key * CPK) * 16u;
        Rsrc k = rk[0], v = rv[0];
#pragma unroll
        for (int w = 1; w < kBN / kPage; ++w)
            if (u == w) k = rk[w], v = rv[w];
        t.k[i] = bld16(k, voff);
        t.v[i] = bld16(v, voff);
    }
}

template <int D, int NT = kThreads, class S = Smem<D>>
__device__ __forceinline__ void store_tile(uint16_t *buf, const TileRegs<D, NT> &t) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < TileRegs<D, NT>::CHUNKS; ++i) {
        const int c = tid + NT * i;
        const int key = c / (D / 8);
        const int d8 = c - key * (D / 8);
        *reinterpret_cast<u32x4 *>(buf + key * S::KSTRIDE + d8 * 8) = t.k[i];
        *reinterpret_cast<u32x4 *>(buf + S::VOFF + key * S::VSTRIDE + d8 * 8) = t.v[i];
    }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read: in each group of 16 lanes, lane 4a+b names
// V[key0 + a][dim0 + 4b .. +3] and lane i of the group receives dims
// dim0 + i at keys key0 .. key0+3 -- one column of V, i.e. a V^T operand.
__device__ __forceinline__ u32x2 ld_tr(const uint16_t *p) {
    const lds_bf16x4 *q = (const lds_bf16x4 *)(__attribute__((address_space(3))) const uint16_t *)p;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)q));
}

// One workgroup of the 32-row kernel: block `bid` of `nblocks`, LDS at smem
// (Smem<D>::BYTES bytes).  Every thread of the workgroup runs it.
template <int D>
__device__ __forceinline__ void prefill32_block(const PrefillArgs &a, int n_qtiles, int bid, int nblocks,
                                                uint16_t *smem) {
    using S = Smem<D>;
    constexpr int KS = D / 16;  // k-steps of the QK contraction
    constexpr int DB = D / 32;  // 32-dim blocks of the output
    constexpr int NS = kBN / 32;  // 32-key score blocks per tile

    // grid: (request, tile, head) with tiles reversed (longest first) and
    // heads fastest, so the G heads of one KV head, which read the same K/V
    // tiles, are G neighbours in that order.  Workgroups are dealt to the 8
    // XCDs round-robin by blockIdx; the remap hands each XCD whole groups of
    // G (groups in order, round-robin over the XCDs), so a group's heads run
    // side by side on one XCD and share its L2, and the order stays longest
    // first.  The last partial round keeps the identity.
    const int G = a.hq / a.hkv;
    int idx = bid;
    if (idx < (nblocks / (8 * G)) * 8 * G) {
        const int k = idx >> 3;
        idx = ((k / G) * 8 + (idx & 7)) * G + k % G;
    }
    const int per_req = n_qtiles * a.hq;
    const int r = idx / per_req;
    const int rem = idx - r * per_req;
    const int qt = n_qtiles - 1 - rem / a.hq;
    const int h = rem - (rem / a.hq) * a.hq;
    // metadata is clamped so that every access stays inside the buffers
    const int q0 = min(max(a.qo_indptr[r], 0), a.total_q);
    const int q_len = min(max(a.qo_indptr[r + 1] - q0, 0), a.total_q - q0);
    if (qt * kBM >= q_len) return;
    const int kv = min(max(a.kv_lens[r], 0), a.max_kv);
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

    // key tiles the workgroup walks; keys every row of this wave sees; the last it needs
    const int i_last_wg = min(qt * kBM + kBM, q_len) - 1;
    const int last_key_wg = a.causal ? kv - q_len + i_last_wg : kv - 1;
    const int n_tiles = last_key_wg / kBN + 1;
    const int wave_first = qt * kBM + wave * kRowsPerWave;
    const int i_last_wave = min(wave_first + kRowsPerWave, q_len) - 1;
    const int last_key_wave = wave_first >= q_len ? -1 : (a.causal ? kv - q_len + i_last_wave : kv - 1);
    const int common_keys = wave_first >= q_len ? -1 : (a.causal ? kv - q_len + wave_first : kv - 1);
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
    // lane's place in the transposing reads of V
    const int grp = lane >> 4;
    const int tr_key = 4 * half + ((lane & 15) >> 2);
    const int tr_dim = 16 * (grp & 1) + 4 * (lane & 3);

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
            const uint16_t *vs = cur + S::TILE;
            // S^T = K . Q^T, one 32x32 block per 32 keys.  K operands are read
            // from LDS in groups (k-steps k0, k0+1 of both key blocks, so
            // consecutive MFMAs alternate accumulators), the next group's reads
            // issued before the current group's MFMAs.
            f32x16 sc[NS];
#pragma unroll
            for (int u = 0; u < NS; ++u) sc[u] = f32x16{};
            constexpr int KG = 2;                 // k-steps per group
            constexpr int GN = NS * KG;           // operands per group
            constexpr int NGRP = KS / KG;
            u32x4 kb[2][GN];
            auto read_group = [&](int gi, u32x4 (&dst)[GN]) {
#pragma unroll
                for (int j = 0; j < GN; ++j) {
                    const int u = j % NS, k = gi * KG + j / NS;
                    dst[j] = *reinterpret_cast<const u32x4 *>(ks + (32 * u + col) * S::STRIDE + 16 * k + 8 * half);
                }
            };
            read_group(0, kb[0]);
#pragma unroll
            for (int gi = 0; gi < NGRP; ++gi) {
                if (gi + 1 < NGRP) read_group(gi + 1, kb[(gi + 1) & 1]);
#pragma unroll
                for (int j = 0; j < GN; ++j) {
                    const int u = j % NS, k = gi * KG + j / NS;
                    sc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kb[gi & 1][j]),
                                                                    __builtin_bit_cast(bf16x8, qop[k]), sc[u], 0, 0,
                                                                    0);
                }
            }
            // scores in log2 units; element e of block u is key tile*64 + 32u + 8(e/4) + 4half + e%4
            float x[NS][16];
            const bool need_mask = tile * kBN + kBN - 1 > common_keys;
            float mx = kNegInff;
#pragma unroll
            for (int u = 0; u < NS; ++u)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    x[u][e] = sc[u][e] * c;
                    if (need_mask) {
                        const int j = tile * kBN + 32 * u + 8 * (e >> 2) + 4 * half + (e & 3);
                        x[u][e] = j <= limit ? x[u][e] : kNegInff;
                    }
                    mx = fmaxf(mx, x[u][e]);
                }
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const bool raise = mx > m + kRescaleSlack;
            if (__any(raise)) {
                const float mn = raise ? mx : m;
                const float alpha = fast_exp2(m - mn);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
                m = mn;
            }
            float sum = 0.f;
            u32x4 pop[2 * NS];
#pragma unroll
            for (int u = 0; u < NS; ++u)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        p[e] = fast_exp2(x[u][8 * t + e] - m);
                        sum += p[e];
                    }
                    pop[2 * u + t] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                           pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
                }
            l += sum;
            // O^T += V^T . P^T; per 16-key step tt: keys 16tt + 4half .. +3 and
            // 16tt + 8 + 4half .. +3.  V^T operands are read (transposing
            // reads) in groups of VG output blocks, the next group's reads
            // issued before the current group's MFMAs.
            constexpr int VG = DB < 4 ? DB : 4;
            constexpr int NVG = 2 * NS * (DB / VG);
            u32x4 vb[2][VG];
            auto read_v = [&](int gi, u32x4 (&dst)[VG]) {
                const int tt = gi / (DB / VG), db0 = (gi % (DB / VG)) * VG;
#pragma unroll
                for (int j = 0; j < VG; ++j) {
                    const uint16_t *base = vs + (16 * tt + tr_key) * S::STRIDE + 32 * (db0 + j) + tr_dim;
                    const u32x2 lo = ld_tr(base);
                    const u32x2 hi = ld_tr(base + 8 * S::STRIDE);
                    dst[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            };
            read_v(0, vb[0]);
#pragma unroll
            for (int gi = 0; gi < NVG; ++gi) {
                if (gi + 1 < NVG) read_v(gi + 1, vb[(gi + 1) & 1]);
                const int tt = gi / (DB / VG), db0 = (gi % (DB / VG)) * VG;
#pragma unroll
                for (int j = 0; j < VG; ++j)
                    acc[db0 + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, vb[gi & 1][j]), __builtin_bit_cast(bf16x8, pop[tt]), acc[db0 + j],
                        0, 0, 0);
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

}  // namespace

}  // namespace pkv
