// route_topk.hip -- top-k expert selection and gate weights, one wavefront
// per token.
//
// Method: ai-from-scratch "19. All-to-all", intro (each token gets a list of
// expert ids) and "Why the router can ruin your day" (the balancing bias
// moves the top-k decision only; the mix weights come from the unbiased
// router scores); aicassindra "gpu_moe_all_to_all", "Two collectives per
// layer" (gate weights scale the returning outputs).
//
// Layout on gfx950: lane l of the wave owns experts l, l + 64, l + 128, ...
// (KPL = ceil(E / 64) registers), so each load instruction reads 256
// contiguous bytes of the logit row. Each selection round takes a wave-wide
// maximum of one 64-bit key per lane -- the lane's best score key in the
// high half and the inverted expert id in the low half, which breaks ties
// towards the smaller id -- then only the owning lane drops the winner and
// refreshes its best. The k results land on lanes 0..k-1, which compute the
// softmax and write one coalesced row of ids and weights.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kTokensPerBlock = kRouteThreads / kWave;

// Order-preserving map of a float score onto uint32: larger key = higher
// rank. -0 and +0 share a key; every NaN maps to 1, below -inf
// (0x007FFFFF); 0 is left for padding lanes and removed entries.
__device__ __forceinline__ uint32_t score_key(float s)
{
    if (s != s)
        return 1u;
    uint32_t u = __float_as_uint(s);
    if ((u << 1) == 0u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int KPL>
struct LaneExperts {
    uint32_t key[KPL];
    float logit[KPL];
    // best entry of this lane: key, expert id, unbiased logit
    uint32_t bk, be;
    float bl;

    __device__ __forceinline__ void refresh_best(int lane)
    {
        bk = 0u;
        be = 0xFFFFFFFFu;
        bl = 0.f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            // ascending i is ascending expert id, so ">" keeps the lower id on ties
            if (key[i] > bk) {
                bk = key[i];
                be = (uint32_t)(i * kWave + lane);
                bl = logit[i];
            }
        }
    }
};

template <int KPL>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int64_t T, int32_t E,
    int32_t k, int normalize, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + (threadIdx.x / kWave);
    if (t >= T)
        return;  // t is uniform across the wave: whole waves leave together
    const float *row = logits + t * E;

    LaneExperts<KPL> le;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = i * kWave + lane;
        if (e < E) {
            const float v = row[e];
            le.logit[i] = v;
            le.key[i] = score_key(bias ? v + bias[e] : v);
        } else {
            le.logit[i] = 0.f;
            le.key[i] = 0u;  // padding ranks below everything, NaN included
        }
    }
    le.refresh_best(lane);

    int32_t my_e = 0;
    float my_l = 0.f;
    float m = -INFINITY;  // max unbiased logit among the selected
    for (int j = 0; j < k; ++j) {
        const uint64_t key = ((uint64_t)le.bk << 32) | (uint32_t)~le.be;
        const uint64_t best = wave_max_u64(key);
        const uint32_t ew = (uint32_t)__builtin_amdgcn_readfirstlane((int)~(uint32_t)best);
        const int owner = (int)(ew & (kWave - 1));
        const int slot = (int)(ew / kWave);
        const float lw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(le.bl), owner));
        if (lane == j) {
            my_e = (int32_t)ew;
            my_l = lw;
        }
        m = fmaxf(m, lw);
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < KPL; ++i)
                if (i == slot)
                    le.key[i] = 0u;
            le.refresh_best(lane);
        }
    }

    float w;
    if (normalize) {
        const float u = lane < k ? expf(my_l - m) : 0.f;
        const float s = wave_sum_f32(u);
        w = u / s;
    } else {
        float lm = -INFINITY;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (i * kWave + lane < E)
                lm = fmaxf(lm, le.logit[i]);
        const float M = wave_max_f32(lm);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (i * kWave + lane < E)
                part += expf(le.logit[i] - M);
        const float s = wave_sum_f32(part);
        w = (lane < k ? expf(my_l - M) : 0.f) / s;
    }
    if (lane < k) {
        topk_idx[t * k + lane] = my_e;
        topk_w[t * k + lane] = w;
    }
}

template <int KPL>
hipError_t launch_kpl(const float *logits, const float *bias, int64_t T, int32_t E, int32_t k,
                      bool normalize, int32_t *topk_idx, float *topk_w, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + kTokensPerBlock - 1) / kTokensPerBlock));
    hipLaunchKernelGGL(route_topk_kernel<KPL>, grid, dim3(kRouteThreads), 0, stream, logits, bias,
                       T, E, k, normalize ? 1 : 0, topk_idx, topk_w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float *logits, const float *bias, int64_t T, int32_t E,
                             int32_t k, bool normalize, int32_t *topk_idx, float *topk_w,
                             hipStream_t stream)
{
    switch ((E + kWave - 1) / kWave) {
#define MOE_ROUTE_CASE(n) \
    case n:               \
        return launch_kpl<n>(logits, bias, T, E, k, normalize, topk_idx, topk_w, stream);
        MOE_ROUTE_CASE(1)
        MOE_ROUTE_CASE(2)
        MOE_ROUTE_CASE(3)
        MOE_ROUTE_CASE(4)
        MOE_ROUTE_CASE(5)
        MOE_ROUTE_CASE(6)
        MOE_ROUTE_CASE(7)
        MOE_ROUTE_CASE(8)
        MOE_ROUTE_CASE(9)
        MOE_ROUTE_CASE(10)
        MOE_ROUTE_CASE(11)
        MOE_ROUTE_CASE(12)
        MOE_ROUTE_CASE(13)
        MOE_ROUTE_CASE(14)
        MOE_ROUTE_CASE(15)
        MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
