// mixed.hip -- chunked prefill and decode rows of one batch in one launch.
//
// The flex-vs-vLLM results page ("What's left on the table", chunked
// prefill) names the separate prefill pass as the main penalty left at large
// batch: a serving step carries both new-prompt chunks (q_r > 1 query rows)
// and decode rows (one query row each) over the same page pool.  Here one
// launch covers both: its grid is one work list whose first workgroups are
// decode split workers (four independent waves each, the decode kernel's
// stream-K cut over the decode rows, see decode.hip) and whose other
// workgroups are the 32-row prefill kernel's (request, query tile, head)
// tiles over the chunks (see prefill.hip).  Decode work comes first: it is the
// latency-critical part of a step, and as its workgroups finish the CUs they
// free take prefill tiles, so the two phases overlap at the boundary instead
// of waiting for each other.  Each row's result is the same softmax
// attention over its visible keys as the separate calls compute (chunk rows
// causal and end-aligned, decode rows over all their keys).
//
// head_dim 64 and 128 (the 4-wave prefill tiles and four decode waves per
// workgroup use the same register budget: one wave per SIMD).
#include <math.h>

#include <atomic>

#include "decode_worker.hpp"
#include "prefill32.hpp"

namespace pkv {

namespace {

template <int D>
struct MixedLds {
    static constexpr int kDecode = kWaves * WorkerLds<D>::kBytes;  // one worker per wave
    static constexpr int kBytes = Smem<D>::BYTES > kDecode ? Smem<D>::BYTES : kDecode;
};

// Blocks 0 .. n_dec_blocks-1: decode workers bid*4 + wave (those at or past
// da.workers do nothing); the rest: prefill tile bid - n_dec_blocks of
// n_pf_blocks.
template <int D, bool SUB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mixed_kernel(PrefillArgs pa, int n_qtiles, int n_pf_blocks, DecodeArgs da, int n_dec_blocks) {
    extern __shared__ __align__(16) uint16_t smem[];
    const int bid = blockIdx.x;
    if (bid < n_dec_blocks) {
        const int wave = uniform((int)threadIdx.x >> 6);
        const int w = bid * kWaves + wave;
        if (w < da.workers)
            decode_bf16_worker<D, SUB>(da, w, reinterpret_cast<char *>(smem) + wave * WorkerLds<D>::kBytes);
        return;
    }
    prefill32_block<D>(pa, n_qtiles, bid - n_dec_blocks, n_pf_blocks, smem);
}

template <int D, bool SUB>
hipError_t launch_mixed_d(const PrefillArgs &pa, const DecodeArgs &da, bool has_decode, hipStream_t stream) {
    const int n_qtiles = pa.batch > 0 ? (pa.max_q + kBM - 1) / kBM : 0;
    const int64_t n_pf = (int64_t)pa.batch * n_qtiles * pa.hq;
    // decode workgroups rounded to whole rounds of the 8 XCDs, so that the
    // prefill tiles keep the XCD grouping their index remap assumes
    int64_t n_dec = has_decode ? (da.workers + kWaves - 1) / kWaves : 0;
    n_dec = (n_dec + 7) / 8 * 8;
    if (n_pf + n_dec > 0x7fffffff) return hipErrorInvalidValue;
    if (n_pf + n_dec == 0) return hipSuccess;
    static std::atomic<uint64_t> attr_set{0};
    hipError_t e =
        set_smem_once(reinterpret_cast<const void *>(&mixed_kernel<D, SUB>), MixedLds<D>::kBytes, attr_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mixed_kernel<D, SUB>), dim3((unsigned)(n_pf + n_dec)), dim3(kThreads), MixedLds<D>::kBytes, stream,
                       pa, n_qtiles, (int)n_pf, da, (int)n_dec);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mixed(const PoolGeom &g, const PrefillArgs &pa, DecodeArgs da, void *workspace, int record_workers,
                        hipStream_t stream) {
    const bool has_decode = da.batch > 0;
    if (has_decode) decode_workspace_layout(g, da, workspace, record_workers);
    const bool sub = g.page_shift > 0;
    switch (g.head_dim) {
        case 64: return sub ? launch_mixed_d<64, true>(pa, da, has_decode, stream)
                            : launch_mixed_d<64, false>(pa, da, has_decode, stream);
        case 128: return sub ? launch_mixed_d<128, true>(pa, da, has_decode, stream)
                             : launch_mixed_d<128, false>(pa, da, has_decode, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
