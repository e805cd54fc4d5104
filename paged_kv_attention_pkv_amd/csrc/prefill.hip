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
// Kernels: one workgroup per (request, tile of 128 or 192 query rows,
// query head); each wave owns 16 query rows of the tile.  Keys are walked in
// tiles of 64 (four 16-token blocks), staged in LDS as [key][dim] rows,
// double-buffered, the next tile's loads in flight during the current one.
// head_dim 256 runs prefill16_kernel, whose tiles move from HBM to LDS by
// buffer-to-LDS transfers; head_dim 64 and 128 run prefill16r_kernel, whose
// tiles pass through registers (their rows need a padded layout that whole
// 1 KB transfers cannot write).  The softmax scale, in log2 units, is applied
// inside exp2 (one fma per score with the max subtracted); Q stays in
// registers for the whole walk; the V^T operand comes straight from the
// [key][dim] rows through gfx950's transposing LDS read.  Keys at or past
// kv_r (tail slots of the last page, which may hold anything) load as zeros
// and masked scores get -inf; tiles that no row of a wave needs are skipped
// and tiles no row's limit cuts are not masked.  Tiles are scheduled longest
// first (causal rows late in a request see the most keys), and whole groups
// of the G query heads of one KV head, which read the same K/V tiles, are
// dealt to one XCD.
//
// The mixed launch (pkv_mixed_attn) runs prefill16r_kernel over one work
// list: the chunks' (request, tile, head) workgroups, then the one-row
// (decode) requests, one workgroup per (request, KV head) computing that KV
// head's G query heads as the rows of one 16-row block.
#include <math.h>

#include <stdint.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {

namespace {

constexpr float kLn2f = 0.6931471805599453f;
constexpr float kNegInff = -__builtin_inff();
// A row's running max is raised only when a tile's scores exceed it by more
// than this (log2 units); weights relative to a stale max stay below 2^8, so
// the output (normalised by the same max) is unchanged and the rescale of the
// accumulators is skipped for most tiles.
constexpr float kRescaleSlack = 8.f;

// ---------------------------------------------------------------------------
// 16 query rows per wave, 8 or 12 waves per workgroup
// ---------------------------------------------------------------------------
//
// Per 64-key tile, with v_mfma_f32_16x16x32_bf16 blocks:
//   S^T[16 key x 16 q]  = K[16 x 32] . Q^T[32 x 16]       (D/32 k-steps per 16 keys)
//   O^T[16 dim x 16 q] += V^T[16 dim x 32 key] . P^T[32 key x 16 q]
// Lane (g = lane/16, c = lane%16) owns query row c of its wave; the softmax
// statistics of a row live in lanes c, c+16, c+32, c+48 (row-swap permutes).
// With 16 rows per wave the accumulators take few registers, so several
// waves share each SIMD and one wave's softmax, barrier wait and LDS reads
// overlap another's MFMAs.
//
// Key order inside a 32-key PV step: lane group g takes keys 4g..4g+3 of the
// first 16-key score block and 4g..4g+3 of the second, which is exactly where
// the S^T accumulators leave them, so P^T needs no data movement; the V^T
// operand is read in the same key order (two transposing reads per block).
//
// Two workgroup sizes (Cfg16): 8 waves (128 query rows, two waves per SIMD)
// and 12 waves (192 rows, three per SIMD, which fits only if a wave stays
// within 168 registers).  Every K/V tile moved into LDS serves all the rows
// of the workgroup, so the 12-wave kernel moves a third fewer bytes per flop
// and has a third more waves to hide LDS latency; on few requests its
// coarser tiles leave CUs idle at the end, and there the 8-wave kernel wins.
// The LDS operand reads of a wave are issued ahead of the MFMAs that use
// them (K: KD k-steps, V^T: VD groups of VG dim blocks), as many as the
// registers allow: a wave alone is bound by LDS latency, not bandwidth.
// At 12 waves the registers are full: the compiler keeps one value that only
// the page-table restage (rows past 65536 keys) uses in scratch memory.
constexpr int kRows16 = 16;
constexpr int kDmaWaves16 = 8;  // waves that issue a tile's transfers
constexpr int kWaves16Max = 12;
template <int W>
struct Cfg16 {
    static_assert(W == 8 || W == 12, "workgroup of 8 or 12 waves");
    static constexpr int WAVES = W;
    static constexpr int THREADS = W * kWave;
    static constexpr int BM = W * kRows16;   // query rows per workgroup
    static constexpr int PER_SIMD = W / 4;    // resident waves per SIMD
    static constexpr int KD = 2;               // k-steps of K reads in flight ahead of the MFMAs
    static constexpr int VG = 2;               // dim blocks per group of V^T reads
    static constexpr int VD = 3;               // groups of V^T reads in flight ahead of the MFMAs
};


typedef __attribute__((address_space(3))) void lds_void;

// Keys per tile and LDS stages of the 16-row kernel (transfers run kNST16-1
// tiles ahead).  64 keys in two stages measured fastest: 32-key tiles in four
// stages (three tiles ahead) lose more to twice the barriers and softmax
// steps than they gain.
constexpr int kBN16 = 64;
constexpr int kNST16 = 2;
static_assert(kBN16 % 32 == 0 && (kNST16 & (kNST16 - 1)) == 0 && kNST16 >= 2 && kNST16 <= 4, "tiling");

// LDS layout of a key tile for the 16-row kernel (D = 256), written by 1 KB
// buffer-to-LDS transfers (64 lanes x 16 B, lane i to byte 16i): key rows in
// pairs, one pair (1 KB) every PAIR elements; the odd row of a pair sits D
// elements after the even one with its 16-byte chunks permuted (chunk j in
// slot j ^ 8).  Measured on the device, both read patterns of the kernel run
// as fast on it as on the best padded row layout.
template <int D>
struct Dma16 {
    static_assert(D == 256, "the row-pair layout is for head_dim 256");
    static constexpr int PAIR = 2 * D + 16;         // elements per row pair (1 KB + 32 B)
    static constexpr int TILE = (kBN16 / 2) * PAIR;  // one of K or V
    static constexpr int BUF = 2 * TILE;             // K then V, one stage
    static constexpr int BYTES = kNST16 * BUF * 2;   // kNST16 stages of bf16
    static constexpr int IDS = kNST16 * BUF;          // then kIds16 int32 table entries (in elements)
    static constexpr int PPW = kBN16 / 16;           // row pairs per wave per tile (K, and V)
    static constexpr int XS = 8;                    // chunk permutation of odd rows
};

// The page of key tile `tile` whose row pairs wave `wave` moves (see dma_tile16).
__device__ __forceinline__ int dma_block16(int tile, int wave) { return tile * (kBN16 / kPage) + ((kBN16 / 16 * wave) >> 3); }

// Table entries are staged in LDS, kIds16 at a time (the blocks of 2 * kIds16
// / (kBN16 / 16) ... tiles), by the whole workgroup (NT threads) before the
// transfers that use them: the compiler cannot tell the LDS transfers from
// stores to the table, so a table read between them would be a vector load
// whose wait covers every transfer in flight.  Entries at or past kv read as 0.
constexpr int kIds16 = 4096;
// Entries are per 16-token block: block j of a row reads table column
// j >> sh (sh = log2(page_size / 16)); its sub-page j & (2^sh - 1) is added
// to the transfer address (dma_tile16).
template <int NT>
__device__ __forceinline__ void stage_ids16(const int32_t *bt, int b0, int kv, int *ids, int sh) {
    constexpr int N = (kIds16 + NT - 1) / NT;
    const int last = (kv - 1) / kPage;  // last block holding a key (kv >= 1 here)
    int v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = bt[min(b0 + (int)threadIdx.x + i * NT, last) >> sh];  // all in flight
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int slot = (int)threadIdx.x + i * NT;
        if (slot < kIds16) ids[slot] = b0 + slot <= last ? v[i] : 0;
    }
}

// The first staging of a row, whose first NT entries (one per thread, `pre`)
// were loaded before the request's lengths were known; the rest of the
// window is loaded here if the row has more blocks.
template <int NT>
__device__ __forceinline__ void stage_ids16_first(const int32_t *bt, int kv, int pre, int *ids, int sh) {
    const int last = (kv - 1) / kPage;  // last block holding a key (kv >= 1 here)
    ids[threadIdx.x] = (int)threadIdx.x <= last ? pre : 0;
    if (last >= NT) {
        constexpr int N = (kIds16 - NT + NT - 1) / NT;
        int v[N];
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = bt[min(NT + (int)threadIdx.x + i * NT, last) >> sh];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int slot = NT + (int)threadIdx.x + i * NT;
            if (slot < kIds16) ids[slot] = slot <= last ? v[i] : 0;
        }
    }
}

// Issue this wave's transfers of key tile `tile` into the stage at dst: wave
// w moves row pairs PPW*w .. PPW*w + PPW-1 of K and of V, which lie in one
// page of the tile (raw table entry `entry`), through that page's buffer
// resource (byte range ending at its last valid key, so keys at or past kv
// land as zeros).  The transfers bypass the registers; the caller waits for
// them (vmcnt) and then for the barrier.
template <int D>
__device__ __forceinline__ void dma_tile16(const PrefillArgs &a, int entry, int g, int tile, int wave, int kv,
                                           uint16_t *dst) {
    using L = Dma16<D>;
    const int lane = threadIdx.x & 63;
    const int64_t tok_bytes = a.s_tok * 2;
    const int blk = dma_block16(tile, wave);
    const int valid = min(max(kv - blk * kPage, 0), kPage);
    int pg = valid > 0 ? entry : 0;
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    // scalar values, so the resources are known to be wave-uniform
    const int64_t sub = blk & ((1 << a.page_shift) - 1);  // 16-token sub-page of a larger page
    const int64_t off = uniform64(((int64_t)pg * a.s_page + (int64_t)g * a.s_head + sub * kPage * a.s_tok) * 2);
    const int32_t bytes = uniform((int)(valid * tok_bytes));
    const Rsrc rk = make_rsrc((const char *)a.k_cache + off, bytes);
    const Rsrc rv = make_rsrc((const char *)a.v_cache + off, bytes);
    const int odd = lane >> 5;                       // second row of the pair
    const int chunk = (lane & 31) ^ (odd * L::XS);   // the global chunk this lane's slot holds
#pragma unroll
    for (int j = 0; j < L::PPW; ++j) {
        const int x = L::PPW * wave + j;  // pair within the tile
        const uint32_t voff = (uint32_t)(((2 * x + odd) & 15) * tok_bytes) + (uint32_t)chunk * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(dst + x * L::PAIR), 16, voff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dst + L::TILE + x * L::PAIR), 16, voff, 0, 0,
                                                 0);
    }
}

// The transposing LDS read (ds_read_b64_tr_b16: in each group of 16 lanes,
// lane 4a+b names V[key0 + a][dim0 + 4b .. +3] and lane i of the group
// receives dims dim0 + i at keys key0 .. key0+3, one column of V), written
// out: for the intrinsic the
// compiler has no alias information, so while buffer-to-LDS transfers are in
// flight it waits for all of them (vmcnt 0) before the read, which would
// drain the transfers running ahead.  Here the read is opaque to the
// compiler: the caller waits for it (lgkm_wait) before using the result.
// The byte offset `off` (a constant once the loops are unrolled) goes into
// the instruction's offset field, so a lane keeps one address register per
// pattern instead of one per read.
__device__ __forceinline__ u32x2 ld_tr_lds(uint32_t lds_byte_addr, uint32_t off) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_byte_addr), "i"(off) : "memory");
    return r;
}

// A 16-byte LDS read written out the same way.  Left to the compiler, the K
// operand reads were hoisted into as many registers as it could find, which
// leaves no room for a third wave per SIMD; written out, the kernel issues
// them exactly KD k-steps ahead.
__device__ __forceinline__ u32x4 ld_lds128(uint32_t lds_byte_addr, uint32_t off) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(lds_byte_addr), "i"(off) : "memory");
    return r;
}

// Wait until at most N LDS reads are in flight, the values in `regs` (the
// results of the reads before those) then being ready; the registers pass
// through the wait so that nothing using them moves above it.
template <int N, int K>
__device__ __forceinline__ void lgkm_wait(u32x4 (&regs)[K]) {
    static_assert(N < 16, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
#pragma unroll
    for (int k = 0; k < K; ++k) asm volatile("" : "+v"(regs[k]));
}

// lgkm_wait with a count n that is a constant once the loops are unrolled.
template <int K>
__device__ __forceinline__ void lgkm_wait_n(int n, u32x4 (&regs)[K]) {
    if (n <= 0) lgkm_wait<0>(regs);
    else if (n == 1) lgkm_wait<1>(regs);
    else if (n == 2) lgkm_wait<2>(regs);
    else if (n == 3) lgkm_wait<3>(regs);
    else if (n == 4) lgkm_wait<4>(regs);
    else if (n == 5) lgkm_wait<5>(regs);
    else if (n == 6) lgkm_wait<6>(regs);
    else if (n == 7) lgkm_wait<7>(regs);
    else if (n == 8) lgkm_wait<8>(regs);
    else if (n == 9) lgkm_wait<9>(regs);
    else if (n == 10) lgkm_wait<10>(regs);
    else if (n == 11) lgkm_wait<11>(regs);
    else if (n == 12) lgkm_wait<12>(regs);
    else if (n == 13) lgkm_wait<13>(regs);
    else lgkm_wait<14>(regs);
}

// Wait until this wave's transfers of the tile after the current one have
// landed while `ahead` later tiles' transfers (TPW per tile) may still run.
// Vector memory operations complete in order; in the s_waitcnt immediate,
// expcnt 7 and lgkmcnt 15 mean no wait on those counters.
template <int TPW>
__device__ __forceinline__ void wait_transfers(int ahead) {
    if constexpr (kNST16 > 2) {
        static_assert(2 * TPW < 16, "vmcnt in the low field");
        if (ahead >= 2)
            __builtin_amdgcn_s_waitcnt((2 * TPW) | 0x0F70);
        else if (ahead == 1)
            __builtin_amdgcn_s_waitcnt(TPW | 0x0F70);
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
        (void)ahead;  // with two stages nothing runs further ahead
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
}

// The scores of a tile enter exp2 as fma(s, c, -m), scaled there, which keeps
// their order only for c > 0.  A negative scale is applied as the negated
// query (bf16 sign bits flipped: every product, and so every score, exactly
// negated) times |c|.  A zero scale is taken as the smallest normal float:
// every weight exp2(s * 2^-126 - m) is then 1 up to rounding for any score
// below 2^100, as with a zero scale.
template <int KS>
__device__ __forceinline__ float positive_scale(float c, u32x4 (&qop)[KS]) {
    if (c < 0.f) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        return -c;
    }
    return c > 0.f ? c : 1.17549435e-38f;
}

// The causal mask on the raw scores of a 64-key tile, and the row's scaled
// maximum on this lane (c > 0).  Element i of block u is key key0 + 16u + i
// (key0 = the tile's first key plus 4 * the lane's group).  The mask runs only
// on tiles that reach past the keys every row of the workgroup sees: as one
// block behind a uniform branch, it stays a branch, where a test per score
// would be turned into index compares and selects on every tile.
template <int NB>
__device__ __forceinline__ float mask_max(f32x4 (&sc)[NB], float c, bool need_mask, int key0, int limit) {
    if (need_mask) {
#pragma unroll
        for (int u = 0; u < NB; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key0 + 16 * u + i > limit) sc[u][i] = kNegInff;
    }
    float mx = kNegInff;
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[u][i]);
    return mx * c;
}

// ---------------------------------------------------------------------------
// key splits
// ---------------------------------------------------------------------------
//
// A call whose (request, query tile, head) workgroups fill the chip at most
// once (few query rows over many keys) may run each of them as S pieces, one
// 8-wave workgroup each (the choice of S is with the launch code below).  Piece s walks key tiles [s*T/S, (s+1)*T/S) of the
// workgroup's T, writes its rows' unnormalised output and (max, sum) as an
// fp32 record and counts itself; the piece that counts last folds the S
// records, its own read back like the others, in piece order and writes the
// rows.  The arithmetic is the same whichever piece is last, so results do
// not depend on the order of arrival.  Records travel between XCDs with
// agent-coherent accesses, like the decode merge's.  A piece's running max
// starts at kSplitFloor instead of -inf: a row whose keys all lie in other
// pieces then gets weights 2^(-inf) = 0, not 2^(-inf + inf).
constexpr float kSplitFloor = -3.0e38f;
constexpr int kMaxSplits = 16;

// Record of piece s of workgroup `unit`: BM x D fp32 output values (in wave
// and lane order, see split_settle), then BM (max, sum) pairs by row.
template <int D, int BM>
__device__ __forceinline__ float *split_record(const PrefillArgs &a, int64_t unit, int s) {
    return a.part + (unit * a.splits + s) * ((int64_t)BM * (D + 2));
}

// After the walk of piece s of workgroup `unit` (every wave of it calls this;
// it synchronises the workgroup): true when this workgroup now holds the
// merged rows (acc, m and lt then cover all the keys), false when another
// piece merges them.  rows: the wave holds query rows of the request (waves
// past its last row neither write nor merge a record); rr: the lane's row in
// the workgroup; lt: the row sum.
//
// The merge's loads go out NR records at a time (NR * D/4 registers of them
// in flight), so that it waits for one round trip to memory per group rather
// than per record; a record is read in the order it was written, each
// instruction 512 contiguous bytes (stored row by row instead, each
// instruction touching 16 rows, the records took 4.7 us to write and 16 us
// to merge at 8 pieces, against 1.4 and 5.5 us in this order; measured per
// workgroup).  Indices past the
// last piece load piece S-1 again and take weight 0, which keeps every
// register index static and the sums' order fixed.
template <int D, int BM>
__device__ bool split_settle(const PrefillArgs &a, int64_t unit, int s, bool rows, int rr, int grp,
                             f32x4 (&acc)[D / 16], float &m, float &lt, int *prior_lds) {
    constexpr int DB = D / 16;
    constexpr int NR = D == 64 ? 4 : 128 / (4 * DB);  // head_dim 64 stays within 128 registers
    const int S = a.splits;
    // record values in wave and lane order: element pair i of dim block db of
    // wave w's lane at ((w * DB + db) * 2 + i) * 128 + 2 * lane, so that each
    // 8-byte store or load instruction covers 512 contiguous bytes
    const int vo = (int)(threadIdx.x >> 6) * DB * 256 + 2 * (int)(threadIdx.x & 63);
    if (rows) {
        float *own = split_record<D, BM>(a, unit, s);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            st_agent2(own + vo + db * 256, acc[db][0], acc[db][1]);
            st_agent2(own + vo + db * 256 + 128, acc[db][2], acc[db][3]);
        }
        if (grp == 0) st_agent2(own + BM * D + rr * 2, m, lt);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the record is complete before the piece counts
    __syncthreads();
    if (threadIdx.x == 0)
        *prior_lds = __hip_atomic_fetch_add(a.arrivals + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*prior_lds != S - 1) return false;
    if (threadIdx.x == 0) __hip_atomic_store(a.arrivals + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!rows) return true;
    // fold the records in piece order, NR per round trip, rescaling the sum
    // so far whenever a group raises the running max
    float M = kSplitFloor, L = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < S; t0 += NR) {
        f32x4 v[NR][DB];
        f32x2 ml[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const float *rec = split_record<D, BM>(a, unit, min(t0 + j, S - 1));
            ml[j] = ld_agent2(rec + BM * D + rr * 2);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x2 lo = ld_agent2(rec + vo + db * 256);
                const f32x2 hi = ld_agent2(rec + vo + db * 256 + 128);
                v[j][db] = f32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
        float Mn = M;
#pragma unroll
        for (int j = 0; j < NR; ++j) Mn = fmaxf(Mn, ml[j][0]);
        const float r = fast_exp2(M - Mn);  // 1 when the max holds, 0 on the first group
        L *= r;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= r;
        M = Mn;
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const float w = t0 + j < S ? fast_exp2(ml[j][0] - M) : 0.f;
            L = fmaf(w, ml[j][1], L);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[db][i] = fmaf(w, v[j][db][i], acc[db][i]);
        }
    }
    m = M;
    lt = L;
    return true;
}

template <int D, int W>
__global__ __launch_bounds__(Cfg16<W>::THREADS) __attribute__((amdgpu_waves_per_eu(Cfg16<W>::PER_SIMD,
                                                                                   Cfg16<W>::PER_SIMD)))
void prefill16_kernel(PrefillArgs a, int n_qtiles) {
    using L = Dma16<D>;
    using C = Cfg16<W>;
    constexpr int kBM16 = C::BM;
    constexpr int KS = D / 32;    // k-steps of the QK contraction
    constexpr int DB = D / 16;    // 16-dim blocks of the output
    constexpr int NB = kBN16 / 16;  // 16-key score blocks per tile
    constexpr int TPW = 2 * Dma16<D>::PPW;  // transfers per wave per tile
    extern __shared__ __align__(16) uint16_t smem[];

    // grid: (request, tile, head) with tiles reversed (longest first) and
    // heads fastest, so the G heads of one KV head, which read the same K/V
    // tiles, are G neighbours in that order.  Workgroups are dealt to the 8
    // XCDs round-robin by blockIdx; the remap hands each XCD whole groups of
    // G (groups in order, round-robin over the XCDs), so a group's heads run
    // side by side on one XCD and share its L2, and the order stays longest
    // first.  The last partial round keeps the identity.
    // With key splits (8-wave instances only) the grid is S copies of that
    // order, piece s of every workgroup in copy s.
    const int G = a.hq / a.hkv;
    int idx = blockIdx.x, nwg = gridDim.x, S = 1, s = 0;
    if constexpr (W == 8) {
        S = a.splits;
        nwg /= S;
        s = idx / nwg;
        idx -= s * nwg;
    }
    if (idx < (nwg / (8 * G)) * 8 * G) {
        const int k = idx >> 3;
        idx = ((k / G) * 8 + (idx & 7)) * G + k % G;
    }
    const int per_req = n_qtiles * a.hq;
    const int r = idx / per_req;
    const int rem = idx - r * per_req;
    const int qt = n_qtiles - 1 - rem / a.hq;
    const int h = rem - (rem / a.hq) * a.hq;
    // the first page-table entries of the row (one per thread) go out before
    // the request's lengths arrive: the row depends only on r
    const int32_t *bt = a.block_table + (int64_t)r * a.bt_cols;
    const int pre_id = ((int)threadIdx.x >> a.page_shift) < a.bt_cols ? bt[(int)threadIdx.x >> a.page_shift] : 0;
    const int q0 = min(max(a.qo_indptr[r], 0), a.total_q);
    const int q_len = min(max(a.qo_indptr[r + 1] - q0, 0), a.total_q - q0);
    if (qt * kBM16 >= q_len) return;
    const int kv = min(max(a.kv_lens[r], 0), a.max_kv);
    const int g = h / G;

    const int wave = uniform(threadIdx.x >> 6);  // scalar: the per-wave tests below are scalar branches
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int i_row = qt * kBM16 + wave * kRows16 + col;
    const bool row_ok = i_row < q_len;
    const int i_eff = row_ok ? i_row : q_len - 1;
    const int limit = a.causal ? kv - q_len + i_eff : kv - 1;

    const int i_last_wg = min(qt * kBM16 + kBM16, q_len) - 1;
    const int last_key_wg = a.causal ? kv - q_len + i_last_wg : kv - 1;
    const int n_tiles = last_key_wg / kBN16 + 1;
    const int t0 = (int)((int64_t)s * n_tiles / S), t1 = (int)((int64_t)(s + 1) * n_tiles / S);  // this piece
    const int wave_first = qt * kBM16 + wave * kRows16;
    const int i_last_wave = min(wave_first + kRows16, q_len) - 1;
    const int last_key_wave = wave_first >= q_len ? -1 : (a.causal ? kv - q_len + i_last_wave : kv - 1);
    const int common_keys = wave_first >= q_len ? -1 : (a.causal ? kv - q_len + wave_first : kv - 1);
    if (kv == 0 || (a.causal && kv < q_len)) {
        if (row_ok) {
            uint16_t *orow = (uint16_t *)a.out + ((int64_t)(q0 + i_row) * a.hq + h) * D;
            for (int d = grp; d < D; d += 4) orow[d] = 0;
            if (grp == 0 && a.lse) a.lse[(int64_t)(q0 + i_row) * a.hq + h] = kNegInff;
        }
        return;
    }

    // Q^T operand: lane holds Q[row][32ks + 8grp .. +7] for every k-step
    u32x4 qop[KS];
    {
        const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)(q0 + i_eff) * a.hq + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = ld16(qrow + 32 * ks + 8 * grp);
    }
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = S > 1 ? kSplitFloor : kNegInff, l = 0.f;  // l: this lane's part of the row sum
    const float c = positive_scale<KS>(a.scale_log2, qop);
    // Lane offsets in the row-pair layout.  A chunk index's bit 3 flips in
    // odd rows, so each pattern has two lane bases: one for reads whose
    // chunk has bit 3 clear (the odd rows' chunk moves up 8) and one for the
    // rest (it moves down 8).
    // K operand: row 16u + col, dims 32k + 8grp (chunk 4k + grp, bit 3 = bit 1 of k)
    const int k_odd = col & 1;
    const int k_base = (col >> 1) * L::PAIR + k_odd * D + 8 * grp;
    const int k_lo = k_base + 64 * k_odd, k_hi = k_base - 64 * k_odd;
    // V^T transposing reads: lane 4a+b of its group names key 32t + 4grp + a
    // (and +16), dims 16db + 4b (chunk 2db + b/2, bit 3 = bit 2 of db)
    const int v_odd = (col >> 2) & 1;
    const int v_base = (2 * grp + (col >> 3)) * L::PAIR + v_odd * D + 8 * ((col & 3) >> 1) + 4 * (col & 1);
    const int v_lo = v_base + 64 * v_odd, v_hi = v_base - 64 * v_odd;

    // table entries of the window holding tile t0 (blocks 0 .. kIds16-1
    // unless a piece starts further on), then tiles t0 .. t0+kNST16-2 in
    // flight, then wait for tile t0
    // waves 0 .. kDmaWaves16-1 issue the transfers
    const int wv = wave;
    int *ids = reinterpret_cast<int *>(smem + L::IDS);
    int window = dma_block16(t0, 0) / kIds16;  // ids holds blocks window*kIds16 ..
    if (window == 0)
        stage_ids16_first<C::THREADS>(bt, kv, pre_id, ids, a.page_shift);
    else
        stage_ids16<C::THREADS>(bt, window * kIds16, kv, ids, a.page_shift);
    // the table in LDS is complete; the Q loads may still be in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    auto entry = [&](int t) { return uniform(ids[dma_block16(t, wv) - window * kIds16]); };
    const int pro = min(kNST16 - 1, t1 - t0);
    if (wv < kDmaWaves16)
        for (int t = t0; t < t0 + pro; ++t)
            dma_tile16<D>(a, entry(t), g, t, wv, kv, smem + (t & (kNST16 - 1)) * L::BUF);
    wait_transfers<TPW>(pro - 1);
    __syncthreads();
    for (int tile = t0; tile < t1; ++tile) {
        uint16_t *cur = smem + (tile & (kNST16 - 1)) * L::BUF;
        const int pre = tile + kNST16 - 1;  // into the stage read in the tile before
        if (pre < t1) {
            // past the staged entries (rows of more than 2 * kIds16 * 16 / (kBN16 / 16) keys): restage,
            // every wave at the same tile; its loads' wait also drains the transfers in flight
            if (dma_block16(pre, kDmaWaves16 - 1) >= (window + 1) * kIds16) {
                __syncthreads();
                window = dma_block16(pre, 0) / kIds16;
                stage_ids16<C::THREADS>(bt, window * kIds16, kv, ids, a.page_shift);
                __syncthreads();
            }
            if (wv < kDmaWaves16)
                dma_tile16<D>(a, entry(pre), g, pre, wv, kv, smem + (pre & (kNST16 - 1)) * L::BUF);
        }

        if (tile * kBN16 <= last_key_wave) {
            const uint16_t *ks = cur;
            const uint16_t *vs = cur + L::TILE;
            // S^T = K . Q^T: per k-step, the NB key blocks' K operands are
            // read together, KD k-steps ahead of the MFMAs that use them
            constexpr int KD = C::KD;
            static_assert(NB * KD <= 15, "LDS read counter");
            f32x4 sc[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            u32x4 kb[KD + 1][NB];
            // raised wave priority while a wave issues MFMAs: when the waves of a
            // SIMD compete for issue, the one feeding the matrix core goes first
            __builtin_amdgcn_s_setprio(1);
            const uint32_t ks_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)ks;
            const uint32_t ka_lo = ks_addr + 2u * (uint32_t)k_lo, ka_hi = ks_addr + 2u * (uint32_t)k_hi;
            auto read_k = [&](int k, u32x4 (&dst)[NB]) {
#pragma unroll
                for (int u = 0; u < NB; ++u)
                    dst[u] = ld_lds128((k & 2) ? ka_hi : ka_lo, 2u * (uint32_t)(8 * u * L::PAIR + 32 * k));
            };
#pragma unroll
            for (int k = 0; k < KD; ++k) read_k(k, kb[k]);
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                // k-step k's reads are done once only the rr later k-steps issued remain
                const int rr = KD - 1 < KS - 1 - k ? KD - 1 : KS - 1 - k;
                lgkm_wait_n(NB * rr, kb[k % (KD + 1)]);
                if (k + KD < KS) read_k(k + KD, kb[(k + KD) % (KD + 1)]);
#pragma unroll
                for (int u = 0; u < NB; ++u)
                    sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[k % (KD + 1)][u]),
                                                                    __builtin_bit_cast(bf16x8, qop[k]), sc[u], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            // raw scores (scaled inside exp2); element i of block u is key tile*64 + 16u + 4grp + i
            const bool need_mask = tile * kBN16 + kBN16 - 1 > common_keys;
            float mx = mask_max<NB>(sc, c, need_mask, tile * kBN16 + 4 * grp, limit);
            mx = rows4_max(mx);
            const bool raise = mx > m + kRescaleSlack;
            if (__any(raise)) {
                const float mn = raise ? mx : m;
                const float alpha = fast_exp2(m - mn);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
                m = mn;
            }
            // P^T operands, one per 32-key step t: keys 4grp.. of blocks 2t and 2t+1
            u32x4 pop[NB / 2];
#pragma unroll
            for (int t = 0; t < NB / 2; ++t) {
                float p[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(fmaf(sc[2 * t][i], c, -m));
                    p[4 + i] = fast_exp2(fmaf(sc[2 * t + 1][i], c, -m));
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) l += p[i];
                pop[t] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7])};
            }
            // O^T += V^T . P^T; V^T operands read in groups of VG dim blocks,
            // VD groups ahead of the MFMAs that use them
            constexpr int VG = C::VG, VD = C::VD;
            static_assert(DB % VG == 0 && 2 * VG * VD <= 15, "LDS read counter");
            constexpr int NVG = (NB / 2) * (DB / VG);
            u32x4 vb[VD + 1][VG];
            __builtin_amdgcn_s_setprio(1);
            // LDS byte addresses of this lane's two V read patterns in the current stage
            const uint32_t vs_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)vs;
            const uint32_t va_lo = vs_addr + 2u * (uint32_t)v_lo, va_hi = vs_addr + 2u * (uint32_t)v_hi;
            auto read_v = [&](int gi, u32x4 (&dst)[VG]) {
                const int t = gi / (DB / VG), db0 = (gi % (DB / VG)) * VG;
#pragma unroll
                for (int j = 0; j < VG; ++j) {
                    const int db = db0 + j;
                    const uint32_t off = 2u * (uint32_t)(16 * t * L::PAIR + 16 * db);
                    const u32x2 lo = ld_tr_lds((db & 4) ? va_hi : va_lo, off);
                    const u32x2 hi = ld_tr_lds((db & 4) ? va_hi : va_lo, off + 2u * 8u * L::PAIR);
                    dst[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            };
#pragma unroll
            for (int gi = 0; gi < VD && gi < NVG; ++gi) read_v(gi, vb[gi]);
#pragma unroll
            for (int gi = 0; gi < NVG; ++gi) {
                // group gi's reads are done once only the rr later groups issued remain
                const int rr = VD - 1 < NVG - 1 - gi ? VD - 1 : NVG - 1 - gi;
                lgkm_wait_n(2 * VG * rr, vb[gi % (VD + 1)]);
                if (gi + VD < NVG) read_v(gi + VD, vb[(gi + VD) % (VD + 1)]);
                const int t = gi / (DB / VG), db0 = (gi % (DB / VG)) * VG;
#pragma unroll
                for (int j = 0; j < VG; ++j)
                    acc[db0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, vb[gi % (VD + 1)][j]), __builtin_bit_cast(bf16x8, pop[t]),
                        acc[db0 + j], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (tile + 1 < t1) {
            // this wave's transfers of the next tile have landed, then every wave's
            wait_transfers<TPW>(min(tile + kNST16 - 1, t1 - 1) - (tile + 1));
            __syncthreads();
        }
    }

    // normalise: acc[db][i] is O^T[dim 16db + 4grp + i][row].  The rows go
    // out through LDS (each wave its own 16-row block, once every wave is
    // done with the tiles), so that each store instruction writes two whole
    // rows instead of touching 16 rows that lie Hq*D*2 bytes apart.  The
    // stores carry the non-temporal hint: nothing in the launch reads the
    // output again, and with the hint a launch that writes 25 MB of it ends
    // ~3 us sooner (measured; the dirty lines otherwise drain from the L2s
    // when the launch ends).
    float lt = rows4_sum(l);
    if constexpr (W == 8) {
        __shared__ int prior;
        if (S > 1 && !split_settle<D, kBM16>(a, ((int64_t)r * n_qtiles + qt) * a.hq + h, s, wave_first < q_len,
                                             wave * kRows16 + col, grp, acc, m, lt, &prior))
            return;
    }
    const float inv = 1.f / lt;
    constexpr int OS = D + 8;  // LDS row stride of the output block (elements)
    static_assert(kWaves16Max * kRows16 * OS * 2 <= Dma16<D>::BYTES, "output block fits the stages");
    __syncthreads();
    uint16_t *ob = smem + wave * kRows16 * OS;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const u32x2 v = {pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv),
                         pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv)};
        *reinterpret_cast<u32x2 *>(ob + col * OS + 16 * db + 4 * grp) = v;
    }
    if (row_ok && grp == 0 && a.lse) a.lse[(int64_t)(q0 + i_row) * a.hq + h] = (m + log2f(lt)) * kLn2f;
    constexpr int LPR = D / 8;        // lanes per row (16 bytes each)
    constexpr int RPI = kWave / LPR;  // rows per store instruction
#pragma unroll
    for (int j = 0; j < kRows16 / RPI; ++j) {
        const int rr = RPI * j + lane / LPR;
        const int ch = lane % LPR;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ob + rr * OS + 8 * ch);
        if (wave_first + rr < q_len)
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4 *>((uint16_t *)a.out + ((int64_t)(q0 + wave_first + rr) * a.hq + h) * D + 8 * ch));
    }
}

// ---------------------------------------------------------------------------
// 16 query rows per wave for head_dim 64 and 128: tiles through registers
// ---------------------------------------------------------------------------
//
// prefill16_kernel's walk (the same MFMA blocks, lane roles, softmax, P^T key
// order and output path) for head_dims whose rows are too short for its
// row-pair transfer layout.  The first 8 waves load each 64-key tile from HBM
// into registers (16-byte chunks, each wave-instruction within one page, so
// one buffer resource per instruction zero-fills keys at or past kv) while the
// tile before is computed, and then write it into the other LDS stage; one
// barrier per tile.  The page-table entries a loading wave needs are read one
// tile earlier still, so no table read waits in front of a tile's loads.
//
// LDS rows are padded to D + 16 elements (288 or 160 bytes).  Measured on the
// device with a probe of the kernel's two read patterns (16 rows x 16 bytes
// per K operand read, 4 rows x 32 bytes per group of a transposing V^T read):
// both run at the conflict-free rate when the row stride is 32 mod 64 bytes,
// and at half that rate or less for strides of 0, 16 or 48 mod 64 and for
// shifted or XOR-swizzled variants of them.
template <int D>
struct Reg16 {
    static_assert(D == 64 || D == 128, "the register-staged 16-row kernel is for head_dim 64 and 128");
    static_assert(((D + 16) * 2) % 64 == 32, "row stride 32 mod 64 bytes");
    static constexpr int RS = D + 16;              // LDS elements per K or V row
    static constexpr int TILE = kBN16 * RS;        // one of K or V
    static constexpr int BUF = 2 * TILE;           // K then V, one stage
    static constexpr int BYTES = kNST16 * BUF * 2;  // kNST16 stages of bf16
    static constexpr int CPK = D / 8;              // 16-byte chunks per key row
    static constexpr int LOADERS = 8;              // waves that load the tiles
    static constexpr int CHUNKS = kBN16 * CPK / (LOADERS * kWave);  // per loading lane, of K and of V
    static constexpr int PAGES = CHUNKS;           // one page per load instruction of a wave
    static_assert(CHUNKS >= 1 && kBN16 * CPK == CHUNKS * LOADERS * kWave, "tile split");
    static_assert(kWave / CPK <= kPage, "a load instruction stays within one page");
};

__device__ __forceinline__ int reg16_row(int r, int rs) { return r * rs; }

template <int D>
struct Reg16Tile {
    u32x4 k[Reg16<D>::CHUNKS], v[Reg16<D>::CHUNKS];
};

// 16-token block of key tile `tile` that load instruction i of loading wave w reads
template <int D>
__device__ __forceinline__ int reg16_block(int tile, int wave, int i) {
    using R = Reg16<D>;
    return tile * (kBN16 / kPage) + ((kWave * wave + R::LOADERS * kWave * i) / R::CPK) / kPage;
}

template <int D>
__device__ __forceinline__ void reg16_load(const PrefillArgs &a, const int (&pg_ids)[Reg16<D>::PAGES], int g,
                                           int tile, int wave, int kv, Reg16Tile<D> &t) {
    using R = Reg16<D>;
    const int lane = threadIdx.x & 63;
    const int64_t tok_bytes = a.s_tok * 2;
#pragma unroll
    for (int i = 0; i < R::CHUNKS; ++i) {
        const int blk = reg16_block<D>(tile, wave, i);
        const int valid = min(max(kv - blk * kPage, 0), kPage);
        int pg = valid > 0 ? pg_ids[i] : 0;
        pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
        const int64_t sub = blk & ((1 << a.page_shift) - 1);
        const int64_t off = uniform64(((int64_t)pg * a.s_page + (int64_t)g * a.s_head + sub * kPage * a.s_tok) * 2);
        const int32_t bytes = uniform((int)(valid * tok_bytes));
        const Rsrc rk = make_rsrc((const char *)a.k_cache + off, bytes);
        const Rsrc rv = make_rsrc((const char *)a.v_cache + off, bytes);
        const int c = kWave * wave + R::LOADERS * kWave * i + lane;  // chunk of the tile
        const int key = c / R::CPK;
        const uint32_t voff = (uint32_t)((key & (kPage - 1)) * tok_bytes) + (uint32_t)(c % R::CPK) * 16u;
        t.k[i] = bld16(rk, voff);
        t.v[i] = bld16(rv, voff);
    }
}

template <int D>
__device__ __forceinline__ void reg16_store(uint16_t *buf, const Reg16Tile<D> &t, int wave) {
    using R = Reg16<D>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < R::CHUNKS; ++i) {
        const int c = kWave * wave + R::LOADERS * kWave * i + lane;
        const int key = c / R::CPK;
        const int e = reg16_row(key, R::RS) + 8 * (c % R::CPK);
        *reinterpret_cast<u32x4 *>(buf + e) = t.k[i];
        *reinterpret_cast<u32x4 *>(buf + R::TILE + e) = t.v[i];
    }
}

// the raw table entries of key tile `tile` for loading wave w (0 past the row's last block)
template <int D>
__device__ __forceinline__ void reg16_ids(const PrefillArgs &a, const int32_t *bt, int tile, int wave, int kv,
                                          int (&ids)[Reg16<D>::PAGES]) {
    const int last = (kv - 1) / kPage;
#pragma unroll
    for (int i = 0; i < Reg16<D>::PAGES; ++i) {
        const int blk = reg16_block<D>(tile, wave, i);
        ids[i] = blk <= last ? bt[blk >> a.page_shift] : 0;
    }
}

template <int D, int W>
__global__ __launch_bounds__(Cfg16<W>::THREADS) __attribute__((amdgpu_waves_per_eu(Cfg16<W>::PER_SIMD,
                                                                                   Cfg16<W>::PER_SIMD)))
void prefill16r_kernel(PrefillArgs a, int n_qtiles, int n_packed, int packed_first) {
    using R = Reg16<D>;
    using C = Cfg16<W>;
    constexpr int kBM16 = C::BM;
    constexpr int KS = D / 32;      // k-steps of the QK contraction
    constexpr int DB = D / 16;      // 16-dim blocks of the output
    constexpr int NB = kBN16 / 16;  // 16-key score blocks per tile
    extern __shared__ __align__(16) uint16_t smem[];

    // The last n_packed workgroups serve one-row requests packed by KV head:
    // packed workgroup p takes request packed_first + p / Hkv and KV head
    // p % Hkv, and its wave 0 computes the G query heads of that KV head as
    // the rows of its 16-row block (lane row c is head g*G + c; every head of
    // a one-row request sees the same keys), the other waves only load tiles.
    // They come after the query tiles (ordered longest first), whose ragged
    // end they fill.  The others: grid as in prefill16_kernel, over requests
    // 0 .. batch-1.
    // With key splits (8-wave instances only) the query-tile part of the
    // grid is S copies of that order, piece s of every workgroup in copy s,
    // and the packed rows follow the last copy.
    const int G = a.hq / a.hkv;
    int n = (int)gridDim.x - n_packed;  // query-tile workgroups
    int bid = (int)blockIdx.x, S = 1, s = 0;
    if constexpr (W == 8) {
        S = a.splits;
        if (S > 1) {
            n /= S;
            if (bid < n * S) {
                s = bid / n;
                bid -= s * n;
            } else {
                bid -= n * (S - 1);
            }
        }
    }
    const bool packed = bid >= n;
    if (packed) S = 1;  // a packed workgroup walks all its keys
    int r, qt, h, g;
    if (packed) {
        const int pk = bid - n;
        r = packed_first + pk / a.hkv;
        g = pk - (r - packed_first) * a.hkv;
        qt = 0;
        h = g * G;
    } else {
        int idx = bid;
        if (idx < (n / (8 * G)) * 8 * G) {
            const int k = idx >> 3;
            idx = ((k / G) * 8 + (idx & 7)) * G + k % G;
        }
        const int per_req = n_qtiles * a.hq;
        r = idx / per_req;
        const int rem = idx - r * per_req;
        qt = n_qtiles - 1 - rem / a.hq;
        h = rem - (rem / a.hq) * a.hq;
        g = h / G;
    }
    const int32_t *bt = a.block_table + (int64_t)r * a.bt_cols;
    const int q0 = min(max(a.qo_indptr[r], 0), a.total_q);
    const int q_len = min(max(a.qo_indptr[r + 1] - q0, 0), a.total_q - q0);
    if (qt * kBM16 >= q_len) return;
    const int kv = min(max(a.kv_lens[r], 0), a.max_kv);

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4;
    const int col = lane & 15;
    // packed: row c of wave 0 is query position 0 of head g*G + c; the other
    // waves hold no row (their first row lies past the request)
    const int head = packed ? h + min(col, G - 1) : h;
    const int i_row = packed ? (wave == 0 && col < G ? 0 : q_len) : qt * kBM16 + wave * kRows16 + col;
    const bool row_ok = i_row < q_len;
    const int i_eff = row_ok ? i_row : q_len - 1;
    const int limit = a.causal ? kv - q_len + i_eff : kv - 1;

    const int i_last_wg = packed ? 0 : min(qt * kBM16 + kBM16, q_len) - 1;
    const int last_key_wg = a.causal ? kv - q_len + i_last_wg : kv - 1;
    const int n_tiles = last_key_wg / kBN16 + 1;
    const int t0 = (int)((int64_t)s * n_tiles / S), t1 = (int)((int64_t)(s + 1) * n_tiles / S);  // this piece
    const int wave_first = packed ? (wave == 0 ? 0 : q_len) : qt * kBM16 + wave * kRows16;
    const int i_last_wave = packed ? 0 : min(wave_first + kRows16, q_len) - 1;
    const int last_key_wave = wave_first >= q_len ? -1 : (a.causal ? kv - q_len + i_last_wave : kv - 1);
    const int common_keys = wave_first >= q_len ? -1 : (a.causal ? kv - q_len + wave_first : kv - 1);
    if (kv == 0 || (a.causal && kv < q_len)) {
        if (row_ok) {
            uint16_t *orow = (uint16_t *)a.out + ((int64_t)(q0 + i_row) * a.hq + head) * D;
            for (int d = grp; d < D; d += 4) orow[d] = 0;
            if (grp == 0 && a.lse) a.lse[(int64_t)(q0 + i_row) * a.hq + head] = kNegInff;
        }
        return;
    }

    const bool loader = wave < R::LOADERS;
    int ids[R::PAGES];
    Reg16Tile<D> regs;
    if (loader && t0 < t1) {
        reg16_ids<D>(a, bt, t0, wave, kv, ids);
        reg16_load<D>(a, ids, g, t0, wave, kv, regs);
        if (t0 + 1 < t1) reg16_ids<D>(a, bt, t0 + 1, wave, kv, ids);
    }
    // Q^T operand: lane holds Q[row][32ks + 8grp .. +7] for every k-step
    u32x4 qop[KS];
    {
        const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)(q0 + i_eff) * a.hq + head) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = ld16(qrow + 32 * ks + 8 * grp);
    }
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = S > 1 ? kSplitFloor : kNegInff, l = 0.f;  // l: this lane's part of the row sum
    const float c = positive_scale<KS>(a.scale_log2, qop);
    // K operand: row 16u + col, dims 32k + 8grp; V^T transposing reads: lane
    // 4a+b of its group names key 32t + 4grp + a (and +16), dims 16db + 4b
    const int k_base = reg16_row(col, R::RS) + 8 * grp;
    const int v_base = reg16_row(4 * grp + (col >> 2), R::RS) + 4 * (col & 3);
    if (loader && t0 < t1) reg16_store<D>(smem + (t0 & 1) * R::BUF, regs, wave);
    __syncthreads();
    for (int tile = t0; tile < t1; ++tile) {
        uint16_t *cur = smem + (tile & 1) * R::BUF;
        uint16_t *nxt = smem + ((tile + 1) & 1) * R::BUF;
        const bool more = tile + 1 < t1;
        if (loader && more) {
            reg16_load<D>(a, ids, g, tile + 1, wave, kv, regs);
            if (tile + 2 < t1) reg16_ids<D>(a, bt, tile + 2, wave, kv, ids);
        }

        if (tile * kBN16 <= last_key_wave) {
            const uint16_t *ks = cur;
            const uint16_t *vs = cur + R::TILE;
            constexpr int KD = C::KD < KS ? C::KD : KS;
            static_assert(NB * KD <= 15, "LDS read counter");
            f32x4 sc[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            u32x4 kb[KD + 1][NB];
            __builtin_amdgcn_s_setprio(1);
            const uint32_t ka = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)ks +
                                2u * (uint32_t)k_base;
            auto read_k = [&](int k, u32x4 (&dst)[NB]) {
#pragma unroll
                for (int u = 0; u < NB; ++u) dst[u] = ld_lds128(ka, 2u * (uint32_t)(16 * u * R::RS + 32 * k));
            };
#pragma unroll
            for (int k = 0; k < KD; ++k) read_k(k, kb[k]);
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int rr = KD - 1 < KS - 1 - k ? KD - 1 : KS - 1 - k;
                lgkm_wait_n(NB * rr, kb[k % (KD + 1)]);
                if (k + KD < KS) read_k(k + KD, kb[(k + KD) % (KD + 1)]);
#pragma unroll
                for (int u = 0; u < NB; ++u)
                    sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[k % (KD + 1)][u]),
                                                                    __builtin_bit_cast(bf16x8, qop[k]), sc[u], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            // raw scores (scaled inside exp2); element i of block u is key tile*64 + 16u + 4grp + i
            const bool need_mask = tile * kBN16 + kBN16 - 1 > common_keys;
            float mx = mask_max<NB>(sc, c, need_mask, tile * kBN16 + 4 * grp, limit);
            mx = rows4_max(mx);
            const bool raise = mx > m + kRescaleSlack;
            if (__any(raise)) {
                const float mn = raise ? mx : m;
                const float alpha = fast_exp2(m - mn);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
                m = mn;
            }
            u32x4 pop[NB / 2];
#pragma unroll
            for (int t = 0; t < NB / 2; ++t) {
                float p[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(fmaf(sc[2 * t][i], c, -m));
                    p[4 + i] = fast_exp2(fmaf(sc[2 * t + 1][i], c, -m));
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) l += p[i];
                pop[t] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7])};
            }
            constexpr int VG = C::VG, VD = C::VD;
            static_assert(DB % VG == 0 && 2 * VG * VD <= 15, "LDS read counter");
            constexpr int NVG = (NB / 2) * (DB / VG);
            u32x4 vb[VD + 1][VG];
            __builtin_amdgcn_s_setprio(1);
            const uint32_t va = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)vs +
                                2u * (uint32_t)v_base;
            auto read_v = [&](int gi, u32x4 (&dst)[VG]) {
                const int t = gi / (DB / VG), db0 = (gi % (DB / VG)) * VG;
#pragma unroll
                for (int j = 0; j < VG; ++j) {
                    const uint32_t off = 2u * (uint32_t)(32 * t * R::RS + 16 * (db0 + j));
                    const u32x2 lo = ld_tr_lds(va, off);
                    const u32x2 hi = ld_tr_lds(va, off + 2u * 16u * R::RS);
                    dst[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            };
#pragma unroll
            for (int gi = 0; gi < VD && gi < NVG; ++gi) read_v(gi, vb[gi]);
#pragma unroll
            for (int gi = 0; gi < NVG; ++gi) {
                const int rr = VD - 1 < NVG - 1 - gi ? VD - 1 : NVG - 1 - gi;
                lgkm_wait_n(2 * VG * rr, vb[gi % (VD + 1)]);
                if (gi + VD < NVG) read_v(gi + VD, vb[(gi + VD) % (VD + 1)]);
                const int t = gi / (DB / VG), db0 = (gi % (DB / VG)) * VG;
#pragma unroll
                for (int j = 0; j < VG; ++j)
                    acc[db0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, vb[gi % (VD + 1)][j]), __builtin_bit_cast(bf16x8, pop[t]),
                        acc[db0 + j], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (more) {
            if (loader) reg16_store<D>(nxt, regs, wave);
            __syncthreads();
        }
    }

    // normalise and write through LDS, as prefill16_kernel
    float lt = rows4_sum(l);
    if constexpr (W == 8) {
        __shared__ int prior;
        if (S > 1 && !split_settle<D, kBM16>(a, ((int64_t)r * n_qtiles + qt) * a.hq + h, s, wave_first < q_len,
                                             wave * kRows16 + col, grp, acc, m, lt, &prior))
            return;
    }
    const float inv = 1.f / lt;
    constexpr int OS = D + 8;
    static_assert(kWaves16Max * kRows16 * OS * 2 <= Reg16<D>::BYTES, "output block fits the stages");
    __syncthreads();
    uint16_t *ob = smem + wave * kRows16 * OS;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const u32x2 v = {pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv),
                         pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv)};
        *reinterpret_cast<u32x2 *>(ob + col * OS + 16 * db + 4 * grp) = v;
    }
    if (row_ok && grp == 0 && a.lse) a.lse[(int64_t)(q0 + i_row) * a.hq + head] = (m + log2f(lt)) * kLn2f;
    constexpr int LPR = D / 8;
    constexpr int RPI = kWave / LPR;
#pragma unroll
    for (int j = 0; j < kRows16 / RPI; ++j) {
        const int rr = RPI * j + lane / LPR;
        const int ch = lane % LPR;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ob + rr * OS + 8 * ch);
        // packed: block row rr is head h + rr of query position 0
        const bool keep = packed ? (wave == 0 && rr < G) : wave_first + rr < q_len;
        const int64_t orow = packed ? (int64_t)q0 * a.hq + h + rr : (int64_t)(q0 + wave_first + rr) * a.hq + h;
        if (keep) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>((uint16_t *)a.out + orow * D + 8 * ch));
    }
}

template <int D, int W>
hipError_t launch16_d(const PrefillArgs &a, hipStream_t stream) {
    constexpr int kSmem16 = Dma16<D>::BYTES + kIds16 * 4;
    constexpr int BM = Cfg16<W>::BM;
    const int n_qtiles = (a.max_q + BM - 1) / BM;
    if (W != 8 && a.splits != 1) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)a.batch * n_qtiles * a.hq * a.splits;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    static std::atomic<uint64_t> attr_set{0};
    hipError_t e = set_smem_once(reinterpret_cast<const void *>(&prefill16_kernel<D, W>), kSmem16, attr_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill16_kernel<D, W>), dim3((unsigned)grid), dim3(Cfg16<W>::THREADS), kSmem16, stream,
                       a, n_qtiles);
    return hipGetLastError();
}

// Query rows per workgroup of the 16-row kernels when the caller leaves the
// choice to the library: 192 once the call has enough 192-row workgroups
// (counted from total_q, which ragged tails only raise), else 128, whose
// finer tiles fill more CUs and end closer together.  head_dim 256: 192 from
// about one and a half rounds on every CU (measured: the single 1023-row
// request, 1.1 rounds, runs faster at 128; two requests of 910 and 627 rows,
// 1.7 rounds, already at 192).  head_dim 64 and 128: 192 above one round
// (measured over 14 shapes: at or under one round 128 is 0-19% faster, e.g.
// one request of 1500 rows 46.8 vs 51.0 us; at 1.1 rounds the two are within
// 1-5%; from 1.4 rounds up 192 is 5-27% faster).
int auto_wg_rows16(const PrefillArgs &a, int head_dim) {
    const int cus = current_device_cus();
    if (cus <= 0) return -1;
    const int64_t wgs192 = ((int64_t)a.total_q + Cfg16<12>::BM - 1) / Cfg16<12>::BM * a.hq;
    if (head_dim != 256) return wgs192 > (int64_t)cus ? Cfg16<12>::BM : Cfg16<8>::BM;
    return 2 * wgs192 >= 3 * (int64_t)cus ? Cfg16<12>::BM : Cfg16<8>::BM;
}

// a.batch requests as (request, tile, head) workgroups, after n_packed_rows
// one-row requests (packed_first ..) as (request, KV head) workgroups
template <int D, int W>
hipError_t launch16r_d(const PrefillArgs &a, hipStream_t stream, int n_packed_rows = 0, int packed_first = 0) {
    constexpr int kSmem = Reg16<D>::BYTES;
    constexpr int BM = Cfg16<W>::BM;
    const int n_qtiles = a.batch > 0 ? (a.max_q + BM - 1) / BM : 0;
    const int64_t n_packed = (int64_t)n_packed_rows * a.hkv;
    if (W != 8 && a.splits != 1) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)a.batch * n_qtiles * a.hq * a.splits + n_packed;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (grid == 0) return hipSuccess;
    static std::atomic<uint64_t> attr_set{0};
    hipError_t e = set_smem_once(reinterpret_cast<const void *>(&prefill16r_kernel<D, W>), kSmem, attr_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill16r_kernel<D, W>), dim3((unsigned)grid), dim3(Cfg16<W>::THREADS), kSmem, stream, a,
                       n_qtiles, (int)n_packed, packed_first);
    return hipGetLastError();
}

// every head_dim runs a 16-row kernel: 256 with its transfer layout, 64 and
// 128 with register-staged tiles
template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t stream) {
    const int rows = a.wg_rows > 0 ? a.wg_rows : auto_wg_rows16(a, D);
    if (rows < 0) return hipErrorInvalidDevice;
    if constexpr (D == 256) {
        if (rows == Cfg16<12>::BM) return launch16_d<D, 12>(a, stream);
        if (rows == Cfg16<8>::BM) return launch16_d<D, 8>(a, stream);
        return hipErrorInvalidValue;
    } else {
        if (rows == Cfg16<12>::BM) return launch16r_d<D, 12>(a, stream);
        if (rows == Cfg16<8>::BM) return launch16r_d<D, 8>(a, stream);
        return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {

// Key splits.  A call whose (request, 128-row query tile, head) workgroups,
// one per CU at a time, fill the chip at most once leaves CUs idle for its
// whole length when it has few of them; with many keys per row it runs
// 8-wave workgroups with each one's key tiles cut into S pieces.  S minimises
// a cost of rounds x piece length: ceil(S x workgroups / CUs) x (ceil(T / S)
// + 8), T = key tiles of the longest row, the 8 tiles standing for a piece's
// start-up, record and merge (~3 + 2 + 5 us, measured per workgroup);
// S <= kMaxSplits, S <= T / 8, at most three rounds of pieces
// (kSplitRounds), ties to the smaller S.  Fitted to sweeps of S = 1 .. 16 on
// 24 shapes (head_dim 64, 128 and 256, 16 to 1023 query rows, 2000 to 32768
// keys, 32 to 384 workgroups): the model's S was within 1.6% of the fastest
// on average and 11% at worst, and 1.3 to 6.7 times faster than no split
// where it splits.  Time falls with S while the pieces fill whole rounds and
// jumps when a round is left part-empty, and each piece slows as more CUs
// run at once; calls of more than one round of workgroups lost with most S
// (the causal q = kv = 1023 request at head_dim 256: 44 us unsplit, 72 at
// S = 2).
constexpr int kSplitRows = Cfg16<8>::BM;
constexpr int kSplitRounds = 3;
constexpr int kSplitPieceCost = 8;  // tiles

int64_t split_units(int batch, int hq, int max_q) {
    return (int64_t)batch * ((max_q + kSplitRows - 1) / kSplitRows) * hq;
}

// The split count for the call, with at most max_pieces pieces in all.
int split_count(int batch, int hq, int max_q, int max_kv, int64_t max_pieces) {
    const int cus = current_device_cus();
    const int64_t units = split_units(batch, hq, max_q);
    if (cus <= 0 || units <= 0 || units > cus) return 1;
    const int64_t tiles = ((int64_t)max_kv + kBN16 - 1) / kBN16;
    const int64_t top = std::min<int64_t>(std::min<int64_t>(tiles / 8, kMaxSplits),
                                          std::min<int64_t>(max_pieces, (int64_t)kSplitRounds * cus) / units);
    int best = 1;
    int64_t best_cost = tiles + kSplitPieceCost;  // S = 1: one round
    for (int64_t S = 2; S <= top; ++S) {
        const int64_t cost = ((S * units + cus - 1) / cus) * ((tiles + S - 1) / S + kSplitPieceCost);
        if (cost < best_cost) {
            best_cost = cost;
            best = (int)S;
        }
    }
    return best;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// bytes: counters (int32 per workgroup), then S records of BM rows x (D + 2) fp32 per workgroup
size_t split_bytes(int head_dim, int64_t units, int splits) {
    return align256((size_t)units * 4) + (size_t)units * splits * kSplitRows * (head_dim + 2) * 4;
}

}  // namespace

size_t prefill_workspace(const PoolGeom &g, int batch, int hq, int total_q, int max_q, int max_kv) {
    (void)total_q;
    if (batch <= 0 || hq <= 0 || max_q <= 0 || max_kv <= 0) return 0;
    const int S = split_count(batch, hq, max_q, max_kv, INT64_MAX);
    return S > 1 ? split_bytes(g.head_dim, split_units(batch, hq, max_q), S) : 0;
}

size_t prefill_split_region_max(int head_dim) {
    // a split call has at most CUs workgroups and kSplitRounds x CUs pieces
    const int cus = current_device_cus();
    if (cus <= 0) return 0;
    return align256((size_t)cus * 4) + (size_t)kSplitRounds * cus * kSplitRows * (head_dim + 2) * 4;
}

namespace {

// Sets a's key-split fields and its 128-row tiling when the call splits its
// keys and `workspace` (zero-filled counters, then records) is large enough;
// otherwise leaves a unsplit and returns false.
bool set_split(const PoolGeom &g, PrefillArgs &a, void *workspace, size_t workspace_bytes) {
    a.splits = 1;
    a.part = nullptr;
    a.arrivals = nullptr;
    if (!workspace || a.batch <= 0 || a.max_q <= 0 || a.max_kv <= 0) return false;
    const int64_t units = split_units(a.batch, a.hq, a.max_q);
    const size_t counters = align256((size_t)units * 4), record = (size_t)kSplitRows * (g.head_dim + 2) * 4;
    if (workspace_bytes < counters + record) return false;
    // the best split whose records fit in the workspace
    const int S = std::min(split_count(a.batch, a.hq, a.max_q, a.max_kv, (workspace_bytes - counters) / record),
                           kMaxSplits);
    if (S <= 1 || workspace_bytes < split_bytes(g.head_dim, units, S)) return false;
    a.splits = S;
    a.arrivals = static_cast<int32_t *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + align256((size_t)units * 4));
    a.wg_rows = kSplitRows;
    return true;
}

template <int D>
hipError_t launch_mixed_d(const PrefillArgs &a, int rows, int n_rows1, int first_row1, hipStream_t stream) {
    if (rows == Cfg16<8>::BM) return launch16r_d<D, 8>(a, stream, n_rows1, first_row1);
    return launch16r_d<D, 12>(a, stream, n_rows1, first_row1);
}

}  // namespace

hipError_t launch_mixed(const PoolGeom &g, const PrefillArgs &args, int n_rows1, int first_row1, void *workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    if (g.head_dim != 64 && g.head_dim != 128) return hipErrorInvalidValue;
    PrefillArgs a = args;
    // the chunks' tiling by pkv_prefill_attn's rule over their own rows, and
    // their key splits as there
    PrefillArgs chunks = a;
    chunks.total_q = a.total_q - n_rows1;
    int rows = auto_wg_rows16(chunks, g.head_dim);
    if (rows < 0) return hipErrorInvalidDevice;
    if (set_split(g, a, workspace, workspace_bytes)) rows = kSplitRows;
    return g.head_dim == 64 ? launch_mixed_d<64>(a, rows, n_rows1, first_row1, stream)
                            : launch_mixed_d<128>(a, rows, n_rows1, first_row1, stream);
}

hipError_t launch_prefill(const PoolGeom &g, const PrefillArgs &args, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    if (args.max_q <= 0 || args.batch <= 0) return hipSuccess;
    PrefillArgs a = args;
    if (a.wg_rows == 0)
        set_split(g, a, workspace, workspace_bytes);
    else
        set_split(g, a, nullptr, 0);
    switch (g.head_dim) {
        case 64: return launch_d<64>(a, stream);
        case 128: return launch_d<128>(a, stream);
        case 256: return launch_d<256>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
