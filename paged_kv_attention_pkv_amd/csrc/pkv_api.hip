// pkv_api.hip -- the C ABI declared in include/pkv.h: host-side argument
// checks, workspace sizing and kernel launches.  No entry point allocates,
// frees, synchronises or reads device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "internal.hpp"
#include "pkv.h"

using pkv::PoolGeom;

namespace {

constexpr int kSub = 16;  // tokens per sub-page, the unit the kernels walk keys in
constexpr int32_t kMaxDecodeKv = 1 << 28;  // decode: max_kv_len bound (PKV_EUNSUPPORTED above)
// Above this max_kv_len the decode rows of a mixed call run as a split decode
// launch beside the chunks' prefill launch.  Packed into one workgroup per
// row and KV head, a decode row walks all its keys alone: with decode rows of
// up to 32768 keys the one launch took 741 us per layer against 331 us for the
// two; with rows of up to 4096 keys the one launch is still faster (244 vs 252).
constexpr int32_t kMixedPackedMaxKv = 8192;
constexpr int32_t kPaddingRow = -1;        // cache length of a padding row (appends and decode steps)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// One KV head's query heads fill at most the 16 columns of an MFMA tile.
bool supported_group(int g) { return g >= 1 && g <= 16; }

// Checks of the descriptor shared by every entry point.
pkv_status check_desc(const pkv_cache_desc *c, PoolGeom *out) {
    if (!c) return PKV_EINVAL;
    if (c->reserved != 0) return PKV_EINVAL;
    if (c->num_pages < 1 || c->num_kv_heads < 1 || c->head_dim < 1 || c->page_size < 1)
        return PKV_EINVAL;
    if (c->s_page < 0 || c->s_head < 0 || c->s_tok < 0) return PKV_EINVAL;
    if (c->dtype != PKV_F32 && c->dtype != PKV_BF16) return PKV_EUNSUPPORTED;
    int shift = -1;
    for (int k = 0; k <= 4; ++k)
        if (c->page_size == (kSub << k)) shift = k;
    if (shift < 0) return PKV_EUNSUPPORTED;  // 16, 32, 64, 128 or 256 tokens per page
    if (((int64_t)c->num_pages << shift) > 0x7fffffff) return PKV_EUNSUPPORTED;  // page ids with their sub-page
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return PKV_EUNSUPPORTED;
    if (c->s_page % 8 || c->s_head % 8 || c->s_tok % 8) return PKV_EUNSUPPORTED;
    // in-page offsets are 32-bit in the kernels
    if (c->s_tok * (int64_t)c->page_size + c->s_head * (int64_t)c->num_kv_heads > (int64_t)1 << 30)
        return PKV_EUNSUPPORTED;
    out->dtype = c->dtype == PKV_BF16 ? 1 : 0;
    out->num_pages = c->num_pages;
    out->page_size = c->page_size;
    out->page_shift = shift;
    out->hkv = c->num_kv_heads;
    out->head_dim = c->head_dim;
    out->s_page = c->s_page;
    out->s_head = c->s_head;
    out->s_tok = c->s_tok;
    return PKV_OK;
}

pkv_status check_heads(const PoolGeom &g, int hq) {
    if (hq < 1 || hq % g.hkv) return PKV_EINVAL;
    if (!supported_group(hq / g.hkv)) return PKV_EUNSUPPORTED;
    return PKV_OK;
}

pkv_status launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ELAUNCH; }

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

void set_msg(char *msg, size_t len, const char *fmt, ...) {
    if (!msg || !len) return;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, len, fmt, ap);
    va_end(ap);
}

int current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    return dev;
}

}  // namespace

constexpr int kMaxDev = 64;  // devices the per-device caches cover

namespace pkv {

namespace {
std::atomic<int> g_cus[kMaxDev];
std::mutex g_attr_mutex;
}  // namespace

int current_device_cus() {
    const int dev = current_device();
    if (dev < 0 || dev >= kMaxDev) return -1;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

hipError_t set_smem_once(const void *kernel, int bytes, std::atomic<uint64_t> &done) {
    const int dev = current_device();
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    const uint64_t bit = 1ull << dev;
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    std::lock_guard<std::mutex> lock(g_attr_mutex);
    if (done.load(std::memory_order_relaxed) & bit) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
    return e;
}

}  // namespace pkv

namespace {

// Device-resident workspace of pkv_append_decode_attn_noalloc, for callers
// that cannot allocate.  Each GPU the library runs on holds its own copy from
// module load until the process ends.  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDev];

// Device address of this device's scratch array (the current device must be
// `dev`), looked up on its first use; nullptr if the lookup fails.
void *scratch_for(int dev) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char *pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "ok";
        case PKV_EINVAL: return "invalid argument";
        case PKV_EUNSUPPORTED: return "unsupported dtype, head_dim, page_size, GQA ratio, stride or alignment";
        case PKV_EWORKSPACE: return "workspace missing or too small";
        case PKV_ELAUNCH: return "kernel launch failed";
        case PKV_EDEVICE: return "no usable HIP device";
        case PKV_EVALIDATE: return "device-data precondition violated";
    }
    return "unknown status";
}

pkv_status pkv_append(const pkv_cache_desc *cache, void *k_cache, void *v_cache, const void *k_new,
                      const void *v_new, const int32_t *block_table, int32_t bt_cols,
                      const int32_t *cache_seqlens, const int32_t *new_indptr, int32_t batch,
                      int32_t total_new, int32_t *seqlens_out, void *stream) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if (batch < 0 || total_new < 0 || bt_cols < 0) return PKV_EINVAL;
    if (batch == 0) return total_new == 0 ? PKV_OK : PKV_EINVAL;
    if (!new_indptr && total_new != batch) return PKV_EINVAL;
    if (!cache_seqlens || (total_new > 0 && (!k_cache || !v_cache || !k_new || !v_new || !block_table ||
                                              bt_cols < 1)))
        return PKV_EINVAL;
    if (seqlens_out && seqlens_out == cache_seqlens) return PKV_EINVAL;
    if (total_new == 0 && !seqlens_out) return PKV_OK;
    if (total_new > 0 &&
        (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new)))
        return PKV_EUNSUPPORTED;
    return launch_status(pkv::launch_append(g, k_cache, v_cache, k_new, v_new, block_table, bt_cols,
                                            cache_seqlens, new_indptr, batch, total_new, seqlens_out,
                                            (hipStream_t)stream));
}

pkv_status pkv_append_rope(const pkv_cache_desc *cache, void *k_cache, void *v_cache, const void *k_new,
                           const void *v_new, void *q, int32_t num_q_heads, const float *rope_cos,
                           const float *rope_sin, int32_t rope_rows, int32_t rope_interleaved,
                           const int32_t *block_table, int32_t bt_cols, const int32_t *cache_seqlens,
                           const int32_t *new_indptr, int32_t batch, int32_t total_new, int32_t *seqlens_out,
                           void *stream) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if (batch < 0 || total_new < 0 || bt_cols < 0 || rope_rows < 0) return PKV_EINVAL;
    if (q && (st = check_heads(g, num_q_heads))) return st;
    if (batch == 0) return total_new == 0 ? PKV_OK : PKV_EINVAL;
    if (!new_indptr && total_new != batch) return PKV_EINVAL;
    if (!cache_seqlens) return PKV_EINVAL;
    if (total_new > 0 && (!k_cache || !v_cache || !k_new || !v_new || !block_table || bt_cols < 1 || !rope_cos ||
                          !rope_sin || rope_rows < 1))
        return PKV_EINVAL;
    if (seqlens_out && seqlens_out == cache_seqlens) return PKV_EINVAL;
    if (total_new == 0 && !seqlens_out) return PKV_OK;
    if (total_new > 0 && (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
                          !aligned16(rope_cos) || !aligned16(rope_sin) || (q && !aligned16(q))))
        return PKV_EUNSUPPORTED;
    return launch_status(pkv::launch_append_rope(g, k_cache, v_cache, k_new, v_new, q, num_q_heads, rope_cos, rope_sin,
                                                 rope_rows, rope_interleaved ? 1 : 0, block_table, bt_cols,
                                                 cache_seqlens, new_indptr, batch, total_new, seqlens_out,
                                                 (hipStream_t)stream));
}

size_t pkv_decode_workspace_bytes_ex(const pkv_cache_desc *cache, int32_t batch, int32_t num_q_heads,
                                     int32_t max_kv_len, int32_t workers) {
    (void)max_kv_len;  // the size does not depend on the lengths
    PoolGeom g;
    if (check_desc(cache, &g) || check_heads(g, num_q_heads) || batch < 1 || workers < 0) return 0;
    const int w = pkv::decode_workers(current_device(), g, num_q_heads, -1, workers);
    if (w < 1) return 0;
    return pkv::decode_workspace(g, batch, num_q_heads, w);
}

size_t pkv_decode_workspace_bytes(const pkv_cache_desc *cache, int32_t batch, int32_t num_q_heads,
                                  int32_t max_kv_len) {
    return pkv_decode_workspace_bytes_ex(cache, batch, num_q_heads, max_kv_len, 0);
}

pkv_status pkv_decode_workspace_reset(const pkv_cache_desc *cache, int32_t batch, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if (batch < 0) return PKV_EINVAL;
    if (batch == 0) return PKV_OK;
    const size_t n = pkv::decode_counter_bytes(g, batch);
    if (!workspace || workspace_bytes < n || !aligned16(workspace)) return PKV_EWORKSPACE;
    return launch_status(pkv::launch_zero_words((int32_t *)workspace, (int64_t)(n / 4), (hipStream_t)stream));
}

}  // extern "C"

namespace {

// What a decode_common call enqueues.
enum class DecodeRun {
    kCall,        // the decode launch, taking a matching plan from the workspace
    kCallNoPlan,  // the decode launch after a clear of the counters, no plan (allocation-free entry)
    kPlan,        // only the plan kernel (q, out, pools, table and new tokens are not used)
};

// Decode, optionally with the step's token appended in the same launch
// (k_new != NULL), or the plan of such calls.
pkv_status decode_common(const pkv_cache_desc *cache, void *out, float *lse, const void *q, int32_t num_q_heads,
                         const void *k_cache, const void *v_cache, const void *k_new, const void *v_new,
                         const int32_t *block_table, int32_t bt_cols, const int32_t *cache_seqlens,
                         int32_t *seqlens_out, int32_t batch, int32_t max_kv_len, float scale, void *workspace,
                         size_t workspace_bytes, int32_t workers, void *stream, DecodeRun run = DecodeRun::kCall,
                         bool plan_fused = false) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if ((st = check_heads(g, num_q_heads))) return st;
    const bool planning = run == DecodeRun::kPlan;
    const bool fused = planning ? plan_fused : (k_new != nullptr || v_new != nullptr);
    if (fused && g.dtype != 1) return PKV_EUNSUPPORTED;
    if (batch < 0 || max_kv_len < 0 || bt_cols < 0 || workers < 0) return PKV_EINVAL;
    if (!planning && fused && (!k_new || !v_new)) return PKV_EINVAL;
    if (seqlens_out && (!fused || seqlens_out == cache_seqlens)) return PKV_EINVAL;
    if (batch == 0) return PKV_OK;
    if (!cache_seqlens) return PKV_EINVAL;
    if (!planning) {
        if (!out || !q || !k_cache || !v_cache || !block_table) return PKV_EINVAL;
        if (fused && (!aligned16(k_new) || !aligned16(v_new))) return PKV_EUNSUPPORTED;
        if ((int64_t)max_kv_len > (int64_t)bt_cols * g.page_size) return PKV_EINVAL;
    }
    if (max_kv_len > kMaxDecodeKv) return PKV_EUNSUPPORTED;  // page counts of 64 rows are summed in 32 bits
    if (!planning) {
        if (!isfinite(scale)) return PKV_EINVAL;
        if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
            return PKV_EUNSUPPORTED;
    }
    const int dev = current_device();
    if (dev < 0) return PKV_EDEVICE;
    // records are laid out for the uncapped count; the launch never has more
    // waves than the call has pages
    const int w_rec = pkv::decode_workers(dev, g, num_q_heads, -1, workers);
    if (w_rec < 1) return PKV_EDEVICE;
    const int64_t bound = (int64_t)batch * g.hkv * ceil_div64(max_kv_len, kSub);
    const int w = bound < w_rec ? (int)(bound > 0 ? bound : 1) : w_rec;
    const size_t need = pkv::decode_workspace(g, batch, num_q_heads, w_rec);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PKV_EWORKSPACE;
    // the fp32 kernel plans at every call: nothing to write
    if (planning && g.dtype != 1) return PKV_OK;

    pkv::DecodeArgs a;
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.s_page = g.s_page;
    a.s_head = g.s_head;
    a.s_tok = g.s_tok;
    a.block_table = block_table;
    a.bt_cols = bt_cols;
    a.seqlens = cache_seqlens;
    a.batch = batch;
    a.hq = num_q_heads;
    a.hkv = g.hkv;
    a.max_kv = max_kv_len;
    a.num_pages = g.num_pages;
    a.page_shift = g.page_shift;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.workers = w;
    a.fixed_workers = workers > 0;
    pkv::decode_mid_cap(dev, g, w_rec, a);
    a.part_o = nullptr;  // filled from the workspace layout at launch
    a.part_ml = nullptr;
    a.arrivals = nullptr;
    a.plan = nullptr;
    a.fused = fused ? 1 : 0;
    a.k_new = k_new;
    a.v_new = v_new;
    a.seqlens_out = seqlens_out;
    if (planning) return launch_status(pkv::launch_decode_plan(g, a, workspace, w_rec, (hipStream_t)stream));
    if (run == DecodeRun::kCallNoPlan) {
        const pkv_status zs = launch_status(pkv::launch_zero_words(
            (int32_t *)workspace, (int64_t)(pkv::decode_counter_bytes(g, batch) / 4), (hipStream_t)stream));
        if (zs) return zs;
    }
    return launch_status(
        pkv::launch_decode(g, a, workspace, w_rec, run == DecodeRun::kCall, (hipStream_t)stream));
}

}  // namespace

extern "C" {

pkv_status pkv_decode_plan(const pkv_cache_desc *cache, int32_t num_q_heads, const int32_t *cache_seqlens,
                           int32_t batch, int32_t max_kv_len, int32_t fused, void *workspace, size_t workspace_bytes,
                           int32_t workers, void *stream) {
    if (fused != 0 && fused != 1) return PKV_EINVAL;
    return decode_common(cache, nullptr, nullptr, nullptr, num_q_heads, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                         cache_seqlens, nullptr, batch, max_kv_len, 1.f, workspace, workspace_bytes, workers, stream,
                         DecodeRun::kPlan, fused == 1);
}

pkv_status pkv_decode_attn_ex(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                              int32_t num_q_heads, const void *k_cache, const void *v_cache,
                              const int32_t *block_table, int32_t bt_cols, const int32_t *cache_seqlens,
                              int32_t batch, int32_t max_kv_len, float scale, void *workspace,
                              size_t workspace_bytes, int32_t workers, void *stream) {
    return decode_common(cache, out, lse, q, num_q_heads, k_cache, v_cache, nullptr, nullptr, block_table,
                         bt_cols, cache_seqlens, nullptr, batch, max_kv_len, scale, workspace, workspace_bytes,
                         workers, stream);
}

pkv_status pkv_append_decode_attn_ex(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                                     int32_t num_q_heads, void *k_cache, void *v_cache, const void *k_new,
                                     const void *v_new, const int32_t *block_table, int32_t bt_cols,
                                     const int32_t *cache_seqlens, int32_t *seqlens_out, int32_t batch,
                                     int32_t max_kv_len, float scale, void *workspace, size_t workspace_bytes,
                                     int32_t workers, void *stream) {
    if (!k_new || !v_new) return PKV_EINVAL;
    return decode_common(cache, out, lse, q, num_q_heads, k_cache, v_cache, k_new, v_new, block_table, bt_cols,
                         cache_seqlens, seqlens_out, batch, max_kv_len, scale, workspace, workspace_bytes, workers,
                         stream);
}

pkv_status pkv_append_decode_attn(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                                  int32_t num_q_heads, void *k_cache, void *v_cache, const void *k_new,
                                  const void *v_new, const int32_t *block_table, int32_t bt_cols,
                                  const int32_t *cache_seqlens, int32_t *seqlens_out, int32_t batch,
                                  int32_t max_kv_len, float scale, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    return pkv_append_decode_attn_ex(cache, out, lse, q, num_q_heads, k_cache, v_cache, k_new, v_new, block_table,
                                     bt_cols, cache_seqlens, seqlens_out, batch, max_kv_len, scale, workspace,
                                     workspace_bytes, 0, stream);
}

pkv_status pkv_append_decode_attn_noalloc(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                                          int32_t num_q_heads, void *k_cache, void *v_cache, const void *k_new,
                                          const void *v_new, const int32_t *block_table, int32_t bt_cols,
                                          const int32_t *cache_seqlens, int32_t *seqlens_out, int32_t batch,
                                          int32_t max_kv_len, float scale, void *stream) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if ((st = check_heads(g, num_q_heads))) return st;
    if (batch < 0) return PKV_EINVAL;
    if (batch == 0) return PKV_OK;
    if (!k_new || !v_new) return PKV_EINVAL;
    const int dev = current_device();
    if (dev < 0 || dev >= kMaxDev) return PKV_EDEVICE;
    const int w_rec = pkv::decode_workers(dev, g, num_q_heads, -1, 0);
    if (w_rec < 1) return PKV_EDEVICE;
    if (pkv::decode_workspace(g, batch, num_q_heads, w_rec) > kScratchBytes)
        return PKV_EWORKSPACE;  // more than the fixed scratch array holds
    void *ws = scratch_for(dev);
    if (!ws) return PKV_EDEVICE;
    // The array keeps the last call's contents: its arrival counters are
    // cleared by a fill kernel on the call's stream before the decode launch.
    return decode_common(cache, out, lse, q, num_q_heads, k_cache, v_cache, k_new, v_new, block_table, bt_cols,
                         cache_seqlens, seqlens_out, batch, max_kv_len, scale, ws, kScratchBytes, 0, stream,
                         DecodeRun::kCallNoPlan);
}

pkv_status pkv_decode_attn(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                           int32_t num_q_heads, const void *k_cache, const void *v_cache,
                           const int32_t *block_table, int32_t bt_cols, const int32_t *cache_seqlens,
                           int32_t batch, int32_t max_kv_len, float scale, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return pkv_decode_attn_ex(cache, out, lse, q, num_q_heads, k_cache, v_cache, block_table, bt_cols,
                              cache_seqlens, batch, max_kv_len, scale, workspace, workspace_bytes, 0,
                              stream);
}

size_t pkv_prefill_workspace_bytes(const pkv_cache_desc *cache, int32_t batch, int32_t num_q_heads,
                                   int32_t total_q, int32_t max_q, int32_t max_kv_len) {
    PoolGeom g;
    if (check_desc(cache, &g) || check_heads(g, num_q_heads) || batch < 1 || total_q < 0 || max_q < 0 ||
        max_kv_len < 0)
        return 0;
    return pkv::prefill_workspace(g, batch, num_q_heads, total_q, max_q, max_kv_len);
}

pkv_status pkv_prefill_attn_ex(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                               int32_t num_q_heads, const void *k_cache, const void *v_cache,
                               const int32_t *block_table, int32_t bt_cols, const int32_t *kv_lens,
                               const int32_t *qo_indptr, int32_t batch, int32_t total_q, int32_t max_q,
                               int32_t max_kv_len, int32_t causal, float scale, void *workspace,
                               size_t workspace_bytes, int32_t rows_per_workgroup, void *stream) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if ((st = check_heads(g, num_q_heads))) return st;
    if (g.dtype != 1) return PKV_EUNSUPPORTED;
    if (batch < 0 || total_q < 0 || max_q < 0 || max_kv_len < 0 || bt_cols < 0) return PKV_EINVAL;
    if (rows_per_workgroup != 0 && rows_per_workgroup != 128 && rows_per_workgroup != 192)
        return PKV_EINVAL;
    if (batch == 0 || total_q == 0) return batch == 0 && total_q != 0 ? PKV_EINVAL : PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !block_table || !kv_lens || !qo_indptr) return PKV_EINVAL;
    if ((int64_t)max_kv_len > (int64_t)bt_cols * g.page_size) return PKV_EINVAL;
    if (!isfinite(scale)) return PKV_EINVAL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_EUNSUPPORTED;
    // a tiling the caller fixed never splits the keys, nor does a call
    // without a workspace; both need none
    const size_t need =
        rows_per_workgroup || !workspace ? 0 : pkv::prefill_workspace(g, batch, num_q_heads, total_q, max_q, max_kv_len);
    if (need && (workspace_bytes < need || !aligned16(workspace))) return PKV_EWORKSPACE;
    pkv::PrefillArgs a;
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.s_page = g.s_page;
    a.s_head = g.s_head;
    a.s_tok = g.s_tok;
    a.block_table = block_table;
    a.bt_cols = bt_cols;
    a.kv_lens = kv_lens;
    a.qo_indptr = qo_indptr;
    a.batch = batch;
    a.hq = num_q_heads;
    a.hkv = g.hkv;
    a.total_q = total_q;
    a.max_q = max_q;
    a.max_kv = max_kv_len;
    a.num_pages = g.num_pages;
    a.page_shift = g.page_shift;
    a.causal = causal ? 1 : 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.wg_rows = rows_per_workgroup;
    a.splits = 1;
    a.part = nullptr;
    a.arrivals = nullptr;
    return launch_status(pkv::launch_prefill(g, a, need ? workspace : nullptr, need ? workspace_bytes : 0,
                                             (hipStream_t)stream));
}

pkv_status pkv_prefill_attn(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                            int32_t num_q_heads, const void *k_cache, const void *v_cache,
                            const int32_t *block_table, int32_t bt_cols, const int32_t *kv_lens,
                            const int32_t *qo_indptr, int32_t batch, int32_t total_q, int32_t max_q,
                            int32_t max_kv_len, int32_t causal, float scale, void *workspace,
                            size_t workspace_bytes, void *stream) {
    return pkv_prefill_attn_ex(cache, out, lse, q, num_q_heads, k_cache, v_cache, block_table, bt_cols, kv_lens,
                               qo_indptr, batch, total_q, max_q, max_kv_len, causal, scale, workspace,
                               workspace_bytes, 0, stream);
}

namespace {

// The mixed workspace: the decode rows' pkv_decode_attn workspace (used when
// they run as their own launch, max_kv_len above kMixedPackedMaxKv), then,
// 256-byte aligned, room for any key split of the chunks.  0: invalid.
size_t mixed_decode_part(const PoolGeom &g, int batch, int num_prefill, int num_q_heads) {
    const int n_dec = batch - num_prefill;
    if (n_dec == 0) return 0;
    const int w = pkv::decode_workers(current_device(), g, num_q_heads, -1, 0);
    if (w < 1) return 0;
    return (pkv::decode_workspace(g, n_dec, num_q_heads, w) + 255) & ~(size_t)255;
}

}  // namespace

size_t pkv_mixed_workspace_bytes(const pkv_cache_desc *cache, int32_t batch, int32_t num_prefill,
                                 int32_t num_q_heads) {
    PoolGeom g;
    if (check_desc(cache, &g) || check_heads(g, num_q_heads) || batch < 1 || num_prefill < 0 || num_prefill > batch)
        return 0;
    const size_t split = pkv::prefill_split_region_max(g.head_dim);
    if (split == 0) return 0;
    if (batch == num_prefill) return split;
    const size_t dec = mixed_decode_part(g, batch, num_prefill, num_q_heads);
    return dec ? dec + split : 0;
}

pkv_status pkv_mixed_attn(const pkv_cache_desc *cache, void *out, float *lse, const void *q, int32_t num_q_heads,
                          const void *k_cache, const void *v_cache, const int32_t *block_table, int32_t bt_cols,
                          const int32_t *kv_lens, const int32_t *qo_indptr, int32_t batch, int32_t num_prefill,
                          int32_t total_q, int32_t max_q, int32_t max_kv_len, float scale, void *workspace,
                          size_t workspace_bytes, void *stream) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if ((st = check_heads(g, num_q_heads))) return st;
    if (g.dtype != 1 || (g.head_dim != 64 && g.head_dim != 128)) return PKV_EUNSUPPORTED;
    if (batch < 0 || num_prefill < 0 || num_prefill > batch || total_q < 0 || max_q < 0 || max_kv_len < 0 ||
        bt_cols < 0)
        return PKV_EINVAL;
    const int n_dec = batch - num_prefill;
    if (total_q < n_dec) return PKV_EINVAL;  // every decode row has one query row
    if (batch == 0) return total_q == 0 ? PKV_OK : PKV_EINVAL;
    if (!out || !q || !k_cache || !v_cache || !block_table || !kv_lens || !qo_indptr) return PKV_EINVAL;
    if ((int64_t)max_kv_len > (int64_t)bt_cols * g.page_size) return PKV_EINVAL;
    if (!isfinite(scale)) return PKV_EINVAL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_EUNSUPPORTED;
    if (current_device() < 0) return PKV_EDEVICE;
    const int64_t pf_rows = (int64_t)total_q - n_dec;

    pkv::PrefillArgs pa;
    pa.q = q;
    pa.out = out;
    pa.lse = lse;
    pa.k_cache = k_cache;
    pa.v_cache = v_cache;
    pa.s_page = g.s_page;
    pa.s_head = g.s_head;
    pa.s_tok = g.s_tok;
    pa.block_table = block_table;
    pa.bt_cols = bt_cols;
    pa.kv_lens = kv_lens;
    pa.qo_indptr = qo_indptr;
    pa.batch = pf_rows > 0 ? num_prefill : 0;  // the chunks, as query tiles
    pa.hq = num_q_heads;
    pa.hkv = g.hkv;
    pa.total_q = total_q;  // chunk rows, then the decode rows' one row each
    pa.max_q = max_q;
    pa.max_kv = max_kv_len;
    pa.num_pages = g.num_pages;
    pa.page_shift = g.page_shift;
    pa.causal = 1;
    pa.scale_log2 = scale * 1.4426950408889634f;
    pa.wg_rows = 0;
    pa.splits = 1;
    pa.part = nullptr;
    pa.arrivals = nullptr;
    // with a workspace: the decode rows' part, then the chunks' key-split region
    size_t dec_bytes = 0;
    void *split_ws = nullptr;
    size_t split_bytes = 0;
    if (workspace) {
        const size_t need = pkv_mixed_workspace_bytes(cache, batch, num_prefill, num_q_heads);
        if (need == 0) return PKV_EDEVICE;
        if (workspace_bytes < need || !aligned16(workspace)) return PKV_EWORKSPACE;
        dec_bytes = mixed_decode_part(g, batch, num_prefill, num_q_heads);
        split_ws = (char *)workspace + dec_bytes;
        split_bytes = workspace_bytes - dec_bytes;
    }
    // Two launches instead of one: the chunks as pkv_prefill_attn, the decode
    // rows (the last n_dec query rows, one each) as pkv_decode_attn, split
    // across workers.  Always for decode rows over more than
    // kMixedPackedMaxKv keys (a packed row is one workgroup per KV head,
    // however long); and, given a workspace, once the packed rows' workgroups
    // (one per row and KV head, each holding a CU for its whole walk) exceed
    // two rounds over the CUs, where the decode kernel's streaming waves
    // finish them sooner (measured over 14 mixes: 128 decode rows at Hkv 8
    // 7-8% faster as two launches, 256 rows 15-18%, 16-64 rows 1-30% slower).
    const int cus = pkv::current_device_cus();
    const bool long_rows = n_dec > 0 && max_kv_len > kMixedPackedMaxKv;
    const bool many_rows = workspace && n_dec > 0 && cus > 0 && (int64_t)n_dec * g.hkv > 2 * (int64_t)cus;
    if (long_rows || many_rows) {
        if (!workspace) return PKV_EWORKSPACE;
        if (pf_rows > 0) {
            pa.batch = num_prefill;
            pa.total_q = (int)pf_rows;
            const pkv_status ps =
                launch_status(pkv::launch_prefill(g, pa, split_ws, split_bytes, (hipStream_t)stream));
            if (ps) return ps;
        }
        const int64_t off = pf_rows * num_q_heads * g.head_dim * 2;  // bytes (bf16)
        return decode_common(cache, (char *)out + off, lse ? lse + pf_rows * num_q_heads : nullptr,
                             (const char *)q + off, num_q_heads, k_cache, v_cache, nullptr, nullptr,
                             block_table + (int64_t)num_prefill * bt_cols, bt_cols, kv_lens + num_prefill, nullptr,
                             n_dec, max_kv_len, scale, workspace, dec_bytes, 0, stream);
    }
    // decode rows: requests num_prefill .. batch-1, one query row each
    return launch_status(pkv::launch_mixed(g, pa, n_dec, num_prefill, split_ws, split_bytes, (hipStream_t)stream));
}

pkv_status pkv_route(const pkv_cache_desc *cache, const int32_t *block_table, int32_t bt_cols,
                     const int32_t *seqlens, int32_t batch, int32_t max_len, int64_t *offsets,
                     void *stream) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if (batch < 0 || max_len < 0 || bt_cols < 0) return PKV_EINVAL;
    if (batch == 0 || max_len == 0) return PKV_OK;
    if (!block_table || !seqlens || !offsets) return PKV_EINVAL;
    if ((int64_t)max_len > (int64_t)bt_cols * g.page_size) return PKV_EINVAL;
    return launch_status(
        pkv::launch_route(g, block_table, bt_cols, seqlens, batch, max_len, offsets, (hipStream_t)stream));
}

pkv_status pkv_validate_host(const pkv_cache_desc *cache, const int32_t *block_table, int32_t bt_cols,
                             const int32_t *kv_lens, const int32_t *qo_indptr, int32_t batch,
                             int32_t total_q, int32_t max_q, int32_t max_kv_len, int32_t causal, char *msg,
                             size_t msg_len) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if (batch < 0 || bt_cols < 0) return PKV_EINVAL;
    if (batch > 0 && (!kv_lens || !block_table)) return PKV_EINVAL;
    if ((int64_t)max_kv_len > (int64_t)bt_cols * g.page_size) {
        set_msg(msg, msg_len, "max_kv_len %d exceeds bt_cols*page_size %lld", max_kv_len,
                (long long)bt_cols * g.page_size);
        return PKV_EVALIDATE;
    }
    for (int b = 0; b < batch; ++b) {
        const int64_t kv = kv_lens[b];
        if (kv < 0 || kv > max_kv_len) {
            set_msg(msg, msg_len, "row %d: kv_len %lld outside 0..max_kv_len (%d)", b, (long long)kv, max_kv_len);
            return PKV_EVALIDATE;
        }
        for (int64_t blk = 0; blk < ceil_div64(kv, g.page_size); ++blk) {
            const int32_t page = block_table[(int64_t)b * bt_cols + blk];
            if (page < 1 || page >= g.num_pages) {
                set_msg(msg, msg_len, "row %d block %lld: page %d not in 1..num_pages-1", b, (long long)blk, page);
                return PKV_EVALIDATE;
            }
        }
    }
    if (qo_indptr) {
        if (qo_indptr[0] != 0 || qo_indptr[batch] != total_q) {
            set_msg(msg, msg_len, "qo_indptr must start at 0 and end at total_q (%d), got %d..%d",
                    total_q, qo_indptr[0], qo_indptr[batch]);
            return PKV_EVALIDATE;
        }
        for (int b = 0; b < batch; ++b) {
            const int64_t ql = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
            if (ql < 0 || ql > max_q || (causal && (ql == 0 || ql > kv_lens[b]))) {
                set_msg(msg, msg_len, "request %d: q_len %lld invalid for kv_len %d", b, (long long)ql, kv_lens[b]);
                return PKV_EVALIDATE;
            }
        }
    }
    if (msg && msg_len) msg[0] = 0;
    return PKV_OK;
}

pkv_status pkv_validate_decode_step_host(const pkv_cache_desc *cache, const int32_t *block_table, int32_t bt_cols,
                                        const int32_t *cache_seqlens, int32_t batch, int32_t max_kv_len, char *msg,
                                        size_t msg_len) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if (batch < 0 || bt_cols < 0) return PKV_EINVAL;
    if (batch > 0 && (!cache_seqlens || !block_table)) return PKV_EINVAL;
    for (int b = 0; b < batch; ++b) {
        if (cache_seqlens[b] == kPaddingRow) continue;
        if (cache_seqlens[b] < 0 || (int64_t)cache_seqlens[b] + 1 > max_kv_len) {
            set_msg(msg, msg_len, "row %d: cached length %d + 1 outside 1..max_kv_len (%d)", b, cache_seqlens[b],
                    max_kv_len);
            return PKV_EVALIDATE;
        }
    }
    // the attended rows (L + 1 keys each) route to real pages ...
    int32_t *attended = (int32_t *)malloc(sizeof(int32_t) * (size_t)(batch > 0 ? batch : 1));
    if (!attended) return PKV_EINVAL;
    for (int b = 0; b < batch; ++b) attended[b] = cache_seqlens[b] == kPaddingRow ? 0 : cache_seqlens[b] + 1;
    st = pkv_validate_host(cache, block_table, bt_cols, attended, nullptr, batch, 0, 0, max_kv_len, 0, msg, msg_len);
    free(attended);
    if (st) return st;
    // ... and no two rows append into the same slot
    return pkv_validate_append_host(cache, block_table, bt_cols, cache_seqlens, nullptr, batch, batch, msg, msg_len);
}

pkv_status pkv_validate_append_host(const pkv_cache_desc *cache, const int32_t *block_table, int32_t bt_cols,
                                    const int32_t *cache_seqlens, const int32_t *new_indptr, int32_t batch,
                                    int32_t total_new, char *msg, size_t msg_len) {
    PoolGeom g;
    pkv_status st = check_desc(cache, &g);
    if (st) return st;
    if (batch < 0 || bt_cols < 0 || total_new < 0) return PKV_EINVAL;
    if (batch > 0 && (!cache_seqlens || !block_table)) return PKV_EINVAL;
    if (new_indptr ? (new_indptr[0] != 0 || new_indptr[batch] != total_new) : total_new != batch) {
        set_msg(msg, msg_len, "new_indptr inconsistent with total_new %d", total_new);
        return PKV_EVALIDATE;
    }
    // (page, slot) targets must be distinct: mark them in a host bitmap
    const size_t slots = (size_t)g.num_pages * g.page_size;
    unsigned char *seen = (unsigned char *)calloc((slots + 7) / 8, 1);
    if (!seen) return PKV_EINVAL;
    pkv_status res = PKV_OK;
    for (int b = 0; b < batch && res == PKV_OK; ++b) {
        const int64_t n_new = new_indptr ? (int64_t)new_indptr[b + 1] - new_indptr[b] : 1;
        if (cache_seqlens[b] == kPaddingRow && n_new >= 0) continue;  // writes nothing
        if (n_new < 0 || cache_seqlens[b] < 0) {
            set_msg(msg, msg_len, "row %d: negative length (%d, %lld)", b, cache_seqlens[b], (long long)n_new);
            res = PKV_EVALIDATE;
            break;
        }
        for (int64_t t = 0; t < n_new; ++t) {
            const int64_t pos = (int64_t)cache_seqlens[b] + t;
            const int64_t blk = pos / g.page_size;
            if (blk >= bt_cols) {
                set_msg(msg, msg_len, "row %d: position %lld beyond the table (%d blocks)", b, (long long)pos, bt_cols);
                res = PKV_EVALIDATE;
                break;
            }
            const int32_t page = block_table[(int64_t)b * bt_cols + blk];
            if (page < 1 || page >= g.num_pages) {
                set_msg(msg, msg_len, "row %d position %lld: page %d not in 1..num_pages-1", b, (long long)pos, page);
                res = PKV_EVALIDATE;
                break;
            }
            const size_t slot = (size_t)page * g.page_size + (size_t)(pos % g.page_size);
            if (seen[slot >> 3] & (1u << (slot & 7))) {
                set_msg(msg, msg_len, "row %d position %lld: slot of page %d written twice", b, (long long)pos, page);
                res = PKV_EVALIDATE;
                break;
            }
            seen[slot >> 3] |= (unsigned char)(1u << (slot & 7));
        }
    }
    free(seen);
    if (res == PKV_OK && msg && msg_len) msg[0] = 0;
    return res;
}

}  // extern "C"
