// device.hpp -- small gfx950 helpers shared by the kernels of this library.
//
// gfx950 runs 64-lane wavefronts; every helper here assumes wave64 and a
// full, converged wave unless it says otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// Row kernels launch one block per row (or token) and x-dimension; past this
// many rows the grid is capped and blocks stride over the rest, which keeps
// grid.x * 256 threads below 2^32.
constexpr int64_t kMaxRowBlocks = (int64_t)1 << 22;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// 64-bit ballot of a predicate across the wave.
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t count_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
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

// DPP lane permutations for wave reductions of commutative, associative
// operations with an identity. Four steps combine pairs, quads, 8-lane
// halves and 16-lane rows (after each step the lanes of a group agree);
// row_bcast:15 then folds row 0 into row 1 and row 2 into row 3, and
// row_bcast:31 folds rows 0-1 into rows 2-3, so lane 63 ends with the whole
// wave's result (lanes 31 and 63 with each 32-lane half's). The association
// order is fixed, so float results are reproducible.
namespace dpp {
constexpr int kQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowHalfMirror = 0x141;  // lane i of 8 <- lane 7 - i
constexpr int kRowMirror = 0x140;      // lane i of 16 <- lane 15 - i
constexpr int kRowBcast15 = 0x142;     // row r <- lane 15 of row r - 1
constexpr int kRowBcast31 = 0x143;     // rows 2, 3 <- lane 31

// lanes of rows outside row_mask read `identity`
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t mov(uint32_t v, uint32_t identity)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xF, false);
}
}  // namespace dpp

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// The compiler's writelane intrinsic, which this clang exposes under no
// builtin name: bound to the intrinsic itself, so instruction selection and
// hazard handling treat it like any other.
__device__ int amdgcn_writelane_i32(int x, int lane, int v) __asm("llvm.amdgcn.writelane.i32");

// v with lane `lane` replaced by the wave-uniform value x (one v_writelane)
__device__ __forceinline__ uint32_t writelane_u32(uint32_t x, int lane, uint32_t v)
{
    return (uint32_t)amdgcn_writelane_i32((int)x, lane, (int)v);
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
