// combine.hip -- inverse permutation and gate-weighted reduction at the
// token's origin, plus the shared expert and the residual.
//
// Method: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
// (expert outputs come back along the inverse permutation, k partial results
// per token, scaled by the router's gate weights); "MoE All-to-All Dispatch
// and Ragged Routing", "Returning Tokens to the Original GPU" (the residual
// add happens where x lives); ai-from-scratch "19. All-to-all", section on
// 512 experts (an always-active shared expert next to the routed ones).
//
// Block (t, y) produces a 4 KiB column slab of out[t]: each lane owns 8
// consecutive elements. The kept rows' positions and weights come in with
// one vector load each (lane j holds entry j) and are broadcast as uniform
// values; all k 16-byte row loads are issued before the first multiply so
// that k loads per lane are in flight. Accumulation is
// float32, one fused multiply-add per kept replica in ascending j, then
// + shared, then + residual, then a single rounding (gfx950's packed
// round-to-nearest-even bf16 convert) or a float32 store.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kRowThreads = 256;

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const u32x4 &v)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_lo(v[q]);
        acc[2 * q + 1] += bf16_hi(v[q]);
    }
}

// KMAX <= kExactK: the kernel is built for exactly k = KMAX replicas, so
// each lane reserves registers for k rows and no more; above it KMAX is a
// bound and k a run-time value.
constexpr int kExactK = 16;

template <int KMAX, bool OUT_F32>
__global__ __launch_bounds__(kRowThreads) void combine_kernel(
    const u32x4 *__restrict__ y, int64_t y_rows, const int32_t *__restrict__ pos,
    const float *__restrict__ topk_w, const u32x4 *__restrict__ shared,
    const u32x4 *__restrict__ residual, int32_t C16, int32_t k_arg, void *__restrict__ out)
{
    const int32_t k = KMAX <= kExactK ? KMAX : k_arg;
    const int64_t t = blockIdx.x;
    const int32_t c = blockIdx.y * kRowThreads + threadIdx.x;
    // the token's k positions and weights: lane j < k of each wave loads entry
    // j (two vector loads in flight at once) and readlane makes each uniform,
    // instead of 2k scalar loads that each wait for the one before. Every lane
    // stays until the broadcasts are done (a lane that left early could not be
    // read).
    const int lane = threadIdx.x & (kWave - 1);
    int32_t pl = -1;
    float wl = 0.f;
    if (lane < k) {
        pl = pos[t * k + lane];
        wl = topk_w[t * k + lane];
    }
    int32_t p[KMAX];
    float wt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        p[j] = -1;
        wt[j] = 0.f;
        if (j < k) {
            const int32_t q = (int32_t)readlane_u32((uint32_t)pl, j);
            if (q >= 0 && q < y_rows) {
                p[j] = q;
                wt[j] = __uint_as_float(readlane_u32(__float_as_uint(wl), j));
            }
        }
    }
    if (c >= C16)
        return;
    u32x4 v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (p[j] >= 0)
            v[j] = load_stream(y + (int64_t)p[j] * C16 + c);
    u32x4 sv = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
    if (shared)
        sv = load_stream(shared + t * C16 + c);
    if (residual)
        rv = load_stream(residual + t * C16 + c);

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (p[j] >= 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(wt[j], bf16_lo(v[j][q]), acc[2 * q]);
                acc[2 * q + 1] = fmaf(wt[j], bf16_hi(v[j][q]), acc[2 * q + 1]);
            }
        }
    }
    if (shared)
        add_bf16x8(acc, sv);
    if (residual)
        add_bf16x8(acc, rv);

    if (OUT_F32) {
        u32x4 *o = reinterpret_cast<u32x4 *>(out) + (t * C16 + c) * 2;
        const u32x4 lo = {__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                          __float_as_uint(acc[2]), __float_as_uint(acc[3])};
        const u32x4 hi = {__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                          __float_as_uint(acc[6]), __float_as_uint(acc[7])};
        o[0] = lo;
        o[1] = hi;
    } else {
        const u32x4 r = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
        reinterpret_cast<u32x4 *>(out)[t * C16 + c] = r;
    }
}

template <int KMAX>
hipError_t launch_kmax(const uint16_t *y, int64_t y_rows, const int32_t *pos, const float *topk_w,
                       const uint16_t *shared, const uint16_t *residual, int64_t T, int32_t H,
                       int32_t k, bool out_fp32, void *out, hipStream_t stream)
{
    const int32_t C16 = H / 8;
    const u32x4 *yv = reinterpret_cast<const u32x4 *>(y);
    // one block per token; past kMaxRowBlocks tokens, one launch per chunk
    for (int64_t t0 = 0; t0 < T; t0 += kMaxRowBlocks) {
        const int64_t n = T - t0 < kMaxRowBlocks ? T - t0 : kMaxRowBlocks;
        const dim3 grid((unsigned)n, (unsigned)((C16 + kRowThreads - 1) / kRowThreads));
        const u32x4 *sv = shared ? reinterpret_cast<const u32x4 *>(shared) + t0 * C16 : nullptr;
        const u32x4 *rv = residual ? reinterpret_cast<const u32x4 *>(residual) + t0 * C16 : nullptr;
        void *o = static_cast<char *>(out) + t0 * C16 * 16 * (out_fp32 ? 2 : 1);
        if (out_fp32)
            hipLaunchKernelGGL((combine_kernel<KMAX, true>), grid, dim3(kRowThreads), 0, stream,
                               yv, y_rows, pos + t0 * k, topk_w + t0 * k, sv, rv, C16, k, o);
        else
            hipLaunchKernelGGL((combine_kernel<KMAX, false>), grid, dim3(kRowThreads), 0, stream,
                               yv, y_rows, pos + t0 * k, topk_w + t0 * k, sv, rv, C16, k, o);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_combine_reduce(const uint16_t *y, int64_t y_rows, const int32_t *pos,
                                 const float *topk_w, const uint16_t *shared,
                                 const uint16_t *residual, int64_t T, int32_t H, int32_t k,
                                 bool out_fp32, void *out, hipStream_t stream)
{
    // one kernel per k up to 16: a kernel built for a bound above k keeps
    // registers for rows it never loads (k = 10 under a bound of 16 took 79
    // VGPRs and 6 waves per SIMD; built for exactly 10, 58 VGPRs and 8)
#define MOE_COMBINE_ARGS y, y_rows, pos, topk_w, shared, residual, T, H, k, out_fp32, out, stream
#define MOE_COMBINE_K(n) \
    case n:              \
        return launch_kmax<n>(MOE_COMBINE_ARGS);
    switch (k) {
        MOE_COMBINE_K(1) MOE_COMBINE_K(2) MOE_COMBINE_K(3) MOE_COMBINE_K(4)
        MOE_COMBINE_K(5) MOE_COMBINE_K(6) MOE_COMBINE_K(7) MOE_COMBINE_K(8)
        MOE_COMBINE_K(9) MOE_COMBINE_K(10) MOE_COMBINE_K(11) MOE_COMBINE_K(12)
        MOE_COMBINE_K(13) MOE_COMBINE_K(14) MOE_COMBINE_K(15) MOE_COMBINE_K(16)
    default:
        return launch_kmax<32>(MOE_COMBINE_ARGS);
    }
#undef MOE_COMBINE_K
#undef MOE_COMBINE_ARGS
}

}  // namespace moe
