// device.hpp -- small gfx950 helpers shared by the kernels of this library.
//
// gfx950 runs 64-lane wavefronts; every helper here assumes wave64 and a
// full, converged wave unless it says otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// 64-bit ballot of a predicate across the wave.
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t count_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int m)
{
    return (uint32_t)__shfl_xor((int)v, m, kWave);
}

// Wave-wide maximum of an unsigned 64-bit value; every lane gets it.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint32_t lo = shfl_xor_u32((uint32_t)v, m);
        uint32_t hi = shfl_xor_u32((uint32_t)(v >> 32), m);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// Wave-wide float sum by an xor butterfly. Lanes i and i^m add the same two
// partial sums at every step, so every lane ends with the same bits and the
// association order is fixed (the result is reproducible).
__device__ __forceinline__ float wave_sum_f32(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// Wave-wide inclusive prefix sum of an int (Hillis-Steele over the lanes).
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int32_t o = __shfl_up(v, d, kWave);
        if (lane >= d)
            v += o;
    }
    return v;
}

// Row-level all-reductions with DPP lane permutations. After the four
// steps every lane of a 16-lane row holds the row's result; every step
// combines two groups whose lanes already agree (pairs, quads, 8-lane
// halves), so the result is the same on every lane of the row and does not
// depend on which lane computes it. The four row results are combined on
// the scalar unit by the callers below.
namespace dpp {
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowHalfMirror = 0x141;  // lane i of 8 <- lane 7 - i
constexpr int kRowMirror = 0x140;      // lane i of 16 <- lane 15 - i

template <int CTRL>
__device__ __forceinline__ uint32_t mov(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
}  // namespace dpp

__device__ __forceinline__ uint32_t row_max_u32(uint32_t v)
{
    v = max(v, dpp::mov<dpp::kQuadSwap1>(v));
    v = max(v, dpp::mov<dpp::kQuadSwap2>(v));
    v = max(v, dpp::mov<dpp::kRowHalfMirror>(v));
    return max(v, dpp::mov<dpp::kRowMirror>(v));
}

__device__ __forceinline__ uint32_t row_min_u32(uint32_t v)
{
    v = min(v, dpp::mov<dpp::kQuadSwap1>(v));
    v = min(v, dpp::mov<dpp::kQuadSwap2>(v));
    v = min(v, dpp::mov<dpp::kRowHalfMirror>(v));
    return min(v, dpp::mov<dpp::kRowMirror>(v));
}

__device__ __forceinline__ float row_sum_f32(float v)
{
    v += __uint_as_float(dpp::mov<dpp::kQuadSwap1>(__float_as_uint(v)));
    v += __uint_as_float(dpp::mov<dpp::kQuadSwap2>(__float_as_uint(v)));
    v += __uint_as_float(dpp::mov<dpp::kRowHalfMirror>(__float_as_uint(v)));
    return v + __uint_as_float(dpp::mov<dpp::kRowMirror>(__float_as_uint(v)));
}

__device__ __forceinline__ float row_max_f32(float v)
{
    v = fmaxf(v, __uint_as_float(dpp::mov<dpp::kQuadSwap1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp::mov<dpp::kQuadSwap2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp::mov<dpp::kRowHalfMirror>(__float_as_uint(v))));
    return fmaxf(v, __uint_as_float(dpp::mov<dpp::kRowMirror>(__float_as_uint(v))));
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Wave-wide results, uniform (held in scalar registers).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = row_max_u32(v);
    return max(max(readlane_u32(v, 0), readlane_u32(v, 16)),
               max(readlane_u32(v, 32), readlane_u32(v, 48)));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = row_min_u32(v);
    return min(min(readlane_u32(v, 0), readlane_u32(v, 16)),
               min(readlane_u32(v, 32), readlane_u32(v, 48)));
}

// Fixed association order: (row0 + row1) + (row2 + row3).
__device__ __forceinline__ float wave_sum_f32_dpp(float v)
{
    v = row_sum_f32(v);
    const uint32_t u = __float_as_uint(v);
    return (__uint_as_float(readlane_u32(u, 0)) + __uint_as_float(readlane_u32(u, 16))) +
           (__uint_as_float(readlane_u32(u, 32)) + __uint_as_float(readlane_u32(u, 48)));
}

__device__ __forceinline__ float wave_max_f32_dpp(float v)
{
    v = row_max_f32(v);
    const uint32_t u = __float_as_uint(v);
    return fmaxf(fmaxf(__uint_as_float(readlane_u32(u, 0)), __uint_as_float(readlane_u32(u, 16))),
                 fmaxf(__uint_as_float(readlane_u32(u, 32)), __uint_as_float(readlane_u32(u, 48))));
}

// bf16 <-> float. A bf16 value is the top half of a float32 pattern, so
// widening is a shift; narrowing uses gfx950's packed convert, which rounds
// to nearest, ties to even, and quiets NaNs.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

// 16 bytes = 8 bf16 values, the unit of every row access.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global accesses. "Streaming" variants set the non-temporal hint
// for data that is touched once and should not displace reusable lines.
__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }

}  // namespace moe
