// common.hpp -- device helpers shared by the libpkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr int kPage = 16;  // tokens per block: pages of 32..256 tokens are walked as runs of 16

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Value of a wave-uniform quantity in a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) { return __shfl_xor(v, mask, kWave); }

// Inclusive prefix sum over the 64 lanes, 32-bit: row_shr steps 1, 2, 4, 8
// inside each 16-lane row (DPP; a lane whose source would lie in another row
// adds 0), then the totals of the rows before (scalar reads of lanes 15, 31,
// 47).  No LDS round trip.
__device__ __forceinline__ int wave_incl_scan32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);
    const int r0 = __builtin_amdgcn_readlane(v, 15);
    const int r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane_id() >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with gfx950's row-swap permutes (VALU, no LDS round trip).  Each swap of a
// value with itself leaves, per lane, the pair {x[l], x[l^16]} (or l^32).
__device__ __forceinline__ float rows4_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t a0 = r[0], a1 = r[1];
    x = fmaxf(__uint_as_float(a0), __uint_as_float(a1));
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t b0 = t[0], b1 = t[1];
    return fmaxf(__uint_as_float(b0), __uint_as_float(b1));
}
__device__ __forceinline__ float rows4_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t a0 = r[0], a1 = r[1];
    x = __uint_as_float(a0) + __uint_as_float(a1);
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t b0 = t[0], b1 = t[1];
    return __uint_as_float(b0) + __uint_as_float(b1);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values to a packed pair of bf16, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// Low 16 bits of a and of b packed as (a.lo, b.lo); likewise for high halves.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// Raw buffer resources (gfx9 descriptor, no stride): a wave-uniform base in
// scalar registers, a 32-bit per-lane byte offset, and a byte range outside
// which loads return zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void *base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// A 16-byte load with the non-temporal hint (data read once).
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ u32x2 ld8_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// fp64 -> bf16 bits, nearest with ties to even, without library calls: the
// value is first rounded to fp32 toward zero with the last bit set when that
// step is inexact (round to odd: fp32 keeps 16 more bits than bf16, so the
// second rounding cannot create a tie or move one), then the fp32 bits are
// rounded to nearest even at bit 16.  Both steps act on bit patterns, so
// fp32 subnormals, overflow to infinity and signed zeros come out as the
// correctly rounded bf16; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_bits_rne(double v) {
    float f = (float)v;  // nearest
    double back = (double)f;
    if (fabs(back) > fabs(v)) {  // rounded away from zero: one step back (|f| > 0 here)
        f = __uint_as_float(__float_as_uint(f) - 1u);
        back = (double)f;
    }
    uint32_t u = __float_as_uint(f);
    if (v != v) return (u >> 16) | 0x40u;
    if (back != v) u |= 1u;  // inexact: round to odd
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Partial results travel between workgroups on different XCDs (each with its
// own L2).  They are written and read with agent-scope atomic accesses,
// which the compiler emits as agent-coherent (sc1) loads and stores, so no
// cache-wide write-back or invalidate (what an agent-scope fence costs on
// this chip) is needed; the writer waits for its stores to complete before
// it announces them with an atomic counter.
__device__ __forceinline__ void st_agent2(float *p, float x, float y) {
    const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, x) | ((uint64_t)__builtin_bit_cast(uint32_t, y) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 ld_agent2(const float *p) {
    const uint64_t v =
        __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x2{__builtin_bit_cast(float, (uint32_t)v), __builtin_bit_cast(float, (uint32_t)(v >> 32))};
}

}  // namespace pkv
