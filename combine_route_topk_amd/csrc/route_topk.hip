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
// contiguous bytes of the logit row. Scores become order-preserving 32-bit
// keys. Each lane keeps its two best remaining (key, id, logit) candidates;
// a selection round is a wave-wide 32-bit maximum (DPP within rows, then
// four readlanes on the scalar unit), a ballot of the lanes holding that
// key, and -- only when two lanes tie on the key -- a wave minimum of their
// expert ids, so ties go to the smaller id. The winning lane pops its
// candidate and rescans its registers only when both candidates are used
// up. Round j's id and logit are kept by lane j, so lanes
// 0..k-1 finish with the softmax and one coalesced row of ids and weights.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kTokensPerBlock = kRouteThreads / kWave;

// Order-preserving map of a float score onto uint32: larger key = higher
// rank. The caller adds +0.0f first, which turns -0 into +0 and leaves
// every other value unchanged, so equal reals get equal keys. Every NaN
// maps to 1, below -inf (0x007FFFFF); 0 marks padding and used entries.
__device__ __forceinline__ uint32_t score_key(float s)
{
    const uint32_t u = __float_as_uint(s);
    const uint32_t k = u ^ (uint32_t)(((int32_t)u >> 31) | (int32_t)0x80000000);
    return s != s ? 1u : k;
}

struct Candidate {
    uint32_t key, id;
    float logit;
};

__device__ __forceinline__ bool ranks_below(uint32_t key, uint32_t id, uint32_t ref_key,
                                            uint32_t ref_id)
{
    return key < ref_key || (key == ref_key && id > ref_id);
}

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

    uint32_t key[KPL];
    float logit[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = i * kWave + lane;
        if (e < E) {
            const float v = row[e];
            logit[i] = v;
            key[i] = score_key((bias ? v + bias[e] : v) + 0.0f);
        } else {
            logit[i] = 0.f;
            key[i] = 0u;
        }
    }

    // the lane's two best entries; ascending i is ascending id, so strict
    // comparisons keep the smaller id first among equal keys
    Candidate c1 = {0u, 0xFFFFFFFFu, 0.f}, c2 = {0u, 0xFFFFFFFFu, 0.f};
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const Candidate c = {key[i], (uint32_t)(i * kWave + lane), logit[i]};
        if (c.key > c1.key) {
            c2 = c1;
            c1 = c;
        } else if (c.key > c2.key) {
            c2 = c;
        }
    }

    uint32_t my_e = 0;
    float my_l = 0.f;
    float m = -INFINITY;  // max unbiased logit among the selected
    for (int j = 0; j < k; ++j) {
        const uint32_t best = wave_max_u32(c1.key);
        const uint64_t holders = ballot64(c1.key == best);
        int owner;
        uint32_t ew;
        if (__popcll(holders) == 1) {
            owner = __ffsll((unsigned long long)holders) - 1;
            ew = readlane_u32(c1.id, owner);
        } else {  // several lanes hold an equal key: the smallest id wins
            ew = wave_min_u32(c1.key == best ? c1.id : 0xFFFFFFFFu);
            owner = (int)(ew & (kWave - 1));
        }
        const float lw = __uint_as_float(readlane_u32(__float_as_uint(c1.logit), owner));
        if (lane == j) {
            my_e = ew;
            my_l = lw;
        }
        m = fmaxf(m, lw);
        if (lane == owner) {
            const uint32_t gone_key = c1.key, gone_id = c1.id;
            c1 = c2;
            c2 = {0u, 0xFFFFFFFFu, 0.f};
            if (c1.key == 0u) {
                // both candidates used: rescan the entries ranked below the
                // last one taken from this lane
#pragma unroll
                for (int i = 0; i < KPL; ++i) {
                    const Candidate c = {key[i], (uint32_t)(i * kWave + lane), logit[i]};
                    if (!ranks_below(c.key, c.id, gone_key, gone_id))
                        continue;
                    if (c.key > c1.key) {
                        c2 = c1;
                        c1 = c;
                    } else if (c.key > c2.key) {
                        c2 = c;
                    }
                }
            }
        }
    }

    float w;
    if (normalize) {
        const float u = lane < k ? expf(my_l - m) : 0.f;
        w = u / wave_sum_f32_dpp(u);
    } else {
        float lm = -INFINITY;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (i * kWave + lane < E)
                lm = fmaxf(lm, logit[i]);
        const float M = wave_max_f32_dpp(lm);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (i * kWave + lane < E)
                part += expf(logit[i] - M);
        w = (lane < k ? expf(my_l - M) : 0.f) / wave_sum_f32_dpp(part);
    }
    if (lane < k) {
        topk_idx[t * k + lane] = (int32_t)my_e;
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
